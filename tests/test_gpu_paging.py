"""GPU tests of expert paging: the device-side slot plan against the
oracle's slot plan (bit-exact: slot maps, stamps, clock hand, fetch list,
slot ids), the fetched slots against the host pages (bit-exact),
and the FFN over the slot pool against the FFN over all experts in device
memory (bit-exact where both take the same kernel plan) and the fp64 oracle
(the FFN's tolerance).  Every call goes through the C ABI."""
import sys

import numpy as np
import pytest
import torch

from nvfp4_routed_expert_amd import native, synth, weights
from oracle import nvfp4_oracle as O
from tests.helpers import LazyOracleExperts, assert_close_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


class DeviceSlots:
    """The slot state on the device, driven through the C ABI."""

    def __init__(self, E, S):
        self.E, self.S = E, S
        i32 = dict(dtype=torch.int32, device=DEV)
        self.slot_of = torch.full((E,), 7, **i32)     # (init must overwrite)
        self.expert_of = torch.full((S,), 7, **i32)
        self.last_use = torch.full((S,), 7, **i32)
        self.hand = torch.full((1,), 7, **i32)
        self.fetch = torch.full((2 * S,), -5, **i32)
        self.n_fetch = torch.zeros(1, **i32)
        P = native._ptr
        native._check(native.lib().moe_expert_cache_init(P(self.slot_of), E, P(self.expert_of),
                                                         P(self.last_use), P(self.hand), S,
                                                         native._stream()))

    def plan(self, ids_np, step, protect_from, max_fetch=None):
        ids = torch.from_numpy(np.ascontiguousarray(ids_np, np.int32)).to(DEV)
        T, k = ids.shape
        slot_ids = torch.full_like(ids, -9)
        P = native._ptr
        mx = self.S if max_fetch is None else max_fetch
        native._check(native.lib().moe_expert_cache_plan(
            P(ids), T, k, self.E, self.S, P(self.slot_of), P(self.expert_of), P(self.last_use),
            P(self.hand), step, protect_from, mx, P(slot_ids), P(self.fetch), P(self.n_fetch),
            native._stream()))
        n = int(self.n_fetch.item())
        f = self.fetch.cpu().numpy()
        return slot_ids.cpu().numpy(), [(int(f[2 * i]), int(f[2 * i + 1])) for i in range(max(n, 0))], n

    def state(self):
        return (self.slot_of.cpu().tolist(), self.expert_of.cpu().tolist(),
                self.last_use.cpu().tolist(), int(self.hand.item()))


def _step_ids(rng, E, T, k, pool, zipf):
    """Ids [T, k] (distinct per token) drawn from `pool` experts of E, with a
    Zipf-like skew over them."""
    subset = rng.choice(E, size=min(pool, E), replace=False)
    p = 1.0 / np.arange(1, len(subset) + 1) ** zipf
    p /= p.sum()
    kk = min(k, len(subset))
    return np.stack([rng.choice(subset, size=kk, replace=False, p=p) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("E,S,k,steps,pool,zipf", [
    (48, 12, 2, 40, 16, 1.0),      # often too full: the failure path
    (128, 64, 8, 30, 40, 0.6),     # decode-shaped
    (64, 64, 4, 12, 64, 0.0),      # pool as large as the expert set
    (1024, 1024, 8, 6, 1024, 0.3),  # the largest state
    (1024, 200, 8, 10, 300, 1.2),
    (1, 1, 1, 4, 1, 0.0),           # one expert, one slot
    (5, 3, 1, 20, 5, 0.5),
])
def test_cache_plan_matches_policy_model(E, S, k, steps, pool, zipf):
    say("cache plan", E, S, k, steps, pool, zipf)
    rng = np.random.default_rng(E * 7 + S)
    dev, ref = DeviceSlots(E, S), O.SlotState(E, S)
    assert dev.state() == (ref.slot_of, ref.expert_of, ref.last_use, ref.hand)
    fails = 0
    for step in range(1, steps + 1):
        T = int(rng.integers(1, 40))
        ids = _step_ids(rng, E, T, k, pool, zipf)
        if step == 3:          # ids outside 0..E-1 are ignored and get slot -1
            ids[0, 0] = -1
            ids[-1, -1] = E
        protect = step - 1 if (step % 2 == 0 and step > 1) else step
        max_fetch = S if step % 3 else max(1, S // 3)   # (a fetch limit below the misses fails)
        got = dev.plan(ids, step, protect, max_fetch)
        want = O.expert_slot_plan(ref, ids, step, protect, max_fetch)
        assert got[2] == want[2], f"step {step}: n_fetch {got[2]} != {want[2]}"
        assert got[1] == want[1], f"step {step}: fetch list"
        assert np.array_equal(got[0], want[0]), f"step {step}: slot ids"
        assert dev.state() == (ref.slot_of, ref.expert_of, ref.last_use, ref.hand), f"step {step}"
        fails += want[2] < 0
    say("plans that did not fit:", fails)
    if (E, S) == (48, 12):
        assert fails > 0


def test_permute_pairs_matches_routing():
    """moe_permute_pairs on routed ids gives moe_route_topk's offsets and
    pair order bit for bit."""
    for T, E, k, zipf in [(37, 8, 2, None), (300, 64, 4, 1.2), (1, 128, 8, None), (700, 256, 8, 1.1)]:
        say("permute", T, E, k, zipf)
        logits = synth.router_logits(T, E, 3, zipf_s=zipf)
        ids, wts, off, pairs = native.moe_route_topk(torch.from_numpy(logits).to(DEV), k)
        off2, pairs2 = native.moe_permute_pairs(ids, E)
        assert torch.equal(off, off2) and torch.equal(pairs, pairs2)


def _host_copy(w):
    return native.ExpertWeights(*[t.cpu().pin_memory() for t in (
        w.gate_codes, w.gate_scales, w.gate_global, w.up_codes, w.up_scales, w.up_global,
        w.down_codes, w.down_scales, w.down_global)])


def _weight_tensors(w):
    return (w.gate_codes, w.gate_scales, w.gate_global, w.up_codes, w.up_scales, w.up_global,
            w.down_codes, w.down_scales, w.down_global)


def _check_pool(cache):
    """Every occupied slot holds its expert's host pages byte for byte."""
    torch.cuda.synchronize()
    eo = cache.expert_of.cpu().tolist()
    occupied = [(s, e) for s, e in enumerate(eo) if e >= 0]
    assert occupied
    ss = torch.tensor([s for s, _ in occupied])
    ee = torch.tensor([e for _, e in occupied])
    for pt, ht in zip(_weight_tensors(cache.pool), _weight_tensors(cache.host)):
        assert torch.equal(pt.cpu()[ss].view(torch.uint8), ht[ee].view(torch.uint8))


def _weights_for(k, T, rng):
    w = rng.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    return w / w.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("T,H,I,E,k,S,pool,protect,bitexact,act", [
    (4, 512, 256, 128, 8, 64, 32, True, True, native.W4A16),   # decode rows: same plan for any E
    (1, 1024, 512, 64, 4, 16, 8, True, True, native.W4A16),
    (300, 256, 256, 64, 2, 64, 64, False, True, native.W4A16),   # tiles, S = E: the same plan
    (200, 256, 128, 64, 2, 40, 40, False, False, native.W4A16),  # tiles, S < E: the tolerance
    (300, 256, 256, 64, 2, 64, 64, False, True, native.W4A4),    # online activation globals
    (200, 256, 128, 64, 2, 40, 40, False, False, native.W4A4),
])
def test_paged_ffn(T, H, I, E, k, S, pool, protect, bitexact, act):
    say("paged ffn", T, H, I, E, k, S, pool, protect, act)
    rng = np.random.default_rng(T + H + E)
    w_dev = weights.synthetic_experts(E, H, I, 5, DEV)
    cache = native.ExpertCache(_host_copy(w_dev), S, DEV)
    for step in range(1, 6):
        ids_np = _step_ids(rng, E, T, k, pool, 0.8)
        wts_np = _weights_for(k, T, rng)
        x = synth.activations(T, H, 100 + step)
        xd = x.to(DEV)
        ids = torch.from_numpy(ids_np).to(DEV)
        wts = torch.from_numpy(wts_np).to(DEV)
        off, pairs = native.moe_permute_pairs(ids, E)
        y_res, g_res = native.moe_grouped_nvfp4_ffn(xd, w_dev, ids, wts, off, pairs, k, act=act,
                                                    out_dtype=torch.float32)
        slot_ids = cache.plan_and_fetch(ids, protect_previous=protect)
        assert int(cache.n_fetch.item()) >= 0, f"step {step}: the step's experts did not fit"
        off_s, pairs_s = native.moe_permute_pairs(slot_ids, S)
        y_pag, g_pag = native.moe_grouped_nvfp4_ffn(xd, cache.pool, slot_ids, wts, off_s, pairs_s,
                                                    k, act=act, out_dtype=torch.float32)
        torch.cuda.synchronize()
        # the slot ids name the same experts
        eo = cache.expert_of.cpu().numpy()
        assert np.array_equal(eo[slot_ids.cpu().numpy()], ids_np), f"step {step}"
        if act == native.W4A4:   # the online globals are maxima over the same values
            assert torch.equal(g_pag, g_res), f"step {step}"
        if bitexact:
            assert torch.equal(y_pag, y_res), f"step {step}"
        else:
            assert_close_f32(y_pag.cpu().numpy(), y_res.cpu().numpy().astype(np.float64),
                             f"paged vs resident, step {step}")
        if step in (1, 5):
            w_ref = LazyOracleExperts(E, H, I, np.unique(ids_np), 5)
            if act == native.W4A4:
                ref, _ = O.moe_ffn(x.float().numpy(), ids_np, wts_np, w_ref, act_quant=True)
            else:
                ref, _ = O.moe_ffn(x.float().numpy(), ids_np, wts_np, w_ref)
            assert_close_f32(y_pag.cpu().numpy(), ref, f"paged vs oracle, step {step}")
    _check_pool(cache)


@pytest.mark.parametrize("workload,S", [("moe_decode", 256), ("moe_prefill", 512)])
def test_paged_ffn_full_size(workload, S):
    """The full-size routed workloads (E = 512, H = 2048, I = 512) on a pool
    of S slots over three routing batches: the paged output equals the
    resident one bit for bit (decode rows at any S; the chunk's tiles with
    S = E take the same plan), the pool equals the host pages."""
    wl = synth.WORKLOADS[workload]
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    say("paged full size", workload, T, H, I, E, k, S)
    w_dev = weights.synthetic_experts(E, H, I, 0, DEV)
    cache = native.ExpertCache(_host_copy(w_dev), S, DEV)
    x = synth.activations(T, H).to(DEV)
    for b in range(3):
        logits = torch.from_numpy(synth.router_logits(T, E, seed=b, zipf_s=wl.zipf_s)).to(DEV)
        ids, wts, off, pairs = native.moe_route_topk(logits, k)
        y_res, _ = native.moe_grouped_nvfp4_ffn(x, w_dev, ids, wts, off, pairs, k,
                                                out_dtype=torch.float32)
        slot_ids = cache.plan_and_fetch(ids)
        off_s, pairs_s = native.moe_permute_pairs(slot_ids, S)
        y_pag, _ = native.moe_grouped_nvfp4_ffn(x, cache.pool, slot_ids, wts, off_s, pairs_s, k,
                                                out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert int(cache.n_fetch.item()) >= 0
        assert torch.equal(y_pag, y_res), f"batch {b}"
    _check_pool(cache)


def test_paged_ffn_two_stream_pipeline():
    """The slot plan, fetch and pair order of step i on a side stream beside
    the FFN of step i-1 on the main stream (the previous step's experts
    protected; the side stream waits for the FFN of step i-2 before reusing
    its buffers): every step's output equals the resident FFN's bit for
    bit (decode row kernels)."""
    T, H, I, E, k, S, steps = 4, 512, 256, 128, 8, 64, 12
    say("paged pipeline", T, H, I, E, k, S, steps)
    rng = np.random.default_rng(11)
    w_dev = weights.synthetic_experts(E, H, I, 6, DEV)
    cache = native.ExpertCache(_host_copy(w_dev), S, DEV)
    xs = [synth.activations(T, H, 200 + i).to(DEV) for i in range(steps)]
    ids_np = [_step_ids(rng, E, T, k, 32, 0.5) for _ in range(steps)]
    wts_np = [_weights_for(k, T, rng) for _ in range(steps)]
    ids_d = [torch.from_numpy(a).to(DEV) for a in ids_np]
    wts_d = [torch.from_numpy(a).to(DEV) for a in wts_np]
    i32 = dict(dtype=torch.int32, device=DEV)
    buf = [dict(slot=torch.empty((T, k), **i32), off=torch.empty(S + 1, **i32),
                pairs=torch.empty(T * k, **i32)) for _ in range(2)]
    nlog = torch.zeros(steps, **i32)
    ws = torch.empty(native.ffn_workspace_bytes(T, H, I, S, k), dtype=torch.uint8, device=DEV)
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs, done = [], []
    side.wait_stream(main)
    for i in range(steps):
        b = buf[i % 2]
        with torch.cuda.stream(side):
            if i >= 2:
                side.wait_event(done[i - 2])
            cache.plan(ids_d[i], protect_previous=True, slot_ids=b["slot"])
            cache.fetch_planned(T * k)
            native.moe_permute_pairs(b["slot"], S, out=(b["off"], b["pairs"]))
            ev = torch.cuda.Event()
            ev.record(side)
            nlog[i:i + 1].copy_(cache.n_fetch)
        main.wait_event(ev)
        y, _ = native.moe_grouped_nvfp4_ffn(xs[i], cache.pool, b["slot"], wts_d[i], b["off"],
                                            b["pairs"], k, out_dtype=torch.float32, workspace=ws)
        outs.append(y)
        d = torch.cuda.Event()
        d.record(main)
        done.append(d)
    main.wait_stream(side)
    torch.cuda.synchronize()
    assert int(nlog.min()) >= 0
    for i in range(steps):
        off, pairs = native.moe_permute_pairs(ids_d[i], E)
        y_res, _ = native.moe_grouped_nvfp4_ffn(xs[i], w_dev, ids_d[i], wts_d[i], off, pairs, k,
                                                out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(outs[i], y_res), f"step {i}"


@pytest.mark.parametrize("T,H,I,E,k,S,act", [
    (4, 512, 256, 64, 4, 8, native.W4A16),      # decode row kernels
    (4, 2048, 512, 64, 4, 8, native.W4A16),     # fused decode FFN
    (4, 512, 256, 64, 4, 8, native.W4A4),       # decode GEMV, online globals
    (300, 256, 256, 64, 2, 8, native.W4A16),    # tiles
    (300, 256, 256, 64, 2, 8, native.W4A4),
])
def test_overfull_plan_drops_unplaced_pairs(T, H, I, E, k, S, act):
    """A step whose experts do not fit the pool: the plan reports -1, moves
    nothing, gives the missing experts' pairs slot id -1 and keeps the hits;
    the FFN on the pool then equals, bit for bit, the resident FFN with those
    pairs dropped (ids -1), tokens without a placed pair are exactly 0, and
    the result matches the oracle with the same pairs dropped."""
    say("over-full plan", T, H, I, E, k, S, act)
    rng = np.random.default_rng(T + E + S)
    w_dev = weights.synthetic_experts(E, H, I, 9, DEV)
    cache = native.ExpertCache(_host_copy(w_dev), S, DEV)
    resident = np.arange(S // 2)                       # step 1 makes these resident
    warm = np.stack([rng.choice(resident, size=min(k, len(resident)), replace=False)
                     for _ in range(T)]).astype(np.int32)
    if warm.shape[1] < k:
        warm = np.concatenate([warm, np.full((T, k - warm.shape[1]), -1, np.int32)], axis=1)
    cache.plan_and_fetch(torch.from_numpy(warm).to(DEV))
    torch.cuda.synchronize()
    assert int(cache.n_fetch.item()) >= 0
    # step 2: hits among the resident experts and more misses than free slots
    misses = np.arange(20, 20 + S + 4)
    ids_np = np.stack([rng.choice(np.concatenate([resident, misses]), size=k, replace=False)
                       for _ in range(T)]).astype(np.int32)
    m = len(misses)   # every miss needed (more than the free slots); token 0 has no placed pair
    for t in range((m + k - 1) // k):
        ids_np[t] = misses[(t * k + np.arange(k)) % m]
    wts_np = _weights_for(k, T, rng)
    before = (cache.slot_of.clone(), cache.expert_of.clone(), cache.hand.clone())
    ids = torch.from_numpy(ids_np).to(DEV)
    slot_ids = cache.plan_and_fetch(ids)
    torch.cuda.synchronize()
    assert int(cache.n_fetch.item()) == -1
    assert all(torch.equal(a, b) for a, b in zip(before, (cache.slot_of, cache.expert_of,
                                                          cache.hand)))
    placed = np.isin(ids_np, resident)
    sid = slot_ids.cpu().numpy()
    assert np.all(sid[~placed] == -1)
    assert np.array_equal(cache.expert_of.cpu().numpy()[sid[placed]], ids_np[placed])
    x = synth.activations(T, H, 42)
    xd = x.to(DEV)
    wts = torch.from_numpy(wts_np).to(DEV)
    off_s, pairs_s = native.moe_permute_pairs(slot_ids, S)
    y_pag, g_pag = native.moe_grouped_nvfp4_ffn(xd, cache.pool, slot_ids, wts, off_s, pairs_s, k,
                                                act=act, out_dtype=torch.float32)
    ids_drop = np.where(placed, ids_np, -1).astype(np.int32)
    idd = torch.from_numpy(ids_drop).to(DEV)
    off, pairs = native.moe_permute_pairs(idd, E)
    y_res, g_res = native.moe_grouped_nvfp4_ffn(xd, w_dev, idd, wts, off, pairs, k, act=act,
                                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    y = y_pag.cpu().numpy()
    assert np.all(y[0] == 0.0)
    if T * k <= 256:   # (the tile plan depends on the expert count: S != E)
        assert torch.equal(y_pag, y_res)
    if act == native.W4A4:
        assert torch.equal(g_pag, g_res)
    assert_close_f32(y, y_res.cpu().numpy().astype(np.float64), "over-full plan vs resident")
    w_ref = LazyOracleExperts(E, H, I, np.unique(ids_np[placed]), 9)
    ref, info = O.moe_ffn(x.float().numpy(), ids_drop, wts_np, w_ref,
                          act_quant=act == native.W4A4)
    if act == native.W4A16:
        assert_close_f32(y, ref, "over-full plan vs oracle")
    else:   # the scales over the kept pairs (g_h: up to a flip of the largest h)
        g = g_pag.cpu().numpy()
        assert g[0] == info["g_x"] and abs(g[1] / info["g_h"] - 1) <= 2 ** -7


def test_fetch_rejects_pageable_host_memory():
    E, H, I = 4, 64, 32
    w_dev = weights.synthetic_experts(E, H, I, 1, DEV)
    pageable = native.ExpertWeights(*[t.cpu() for t in _weight_tensors(w_dev)])
    with pytest.raises(ValueError):
        native.ExpertCache(pageable, 2, DEV)
    pool = weights.empty_experts(2, H, I, DEV)
    fetch = torch.zeros(4, dtype=torch.int32, device=DEV)
    n = torch.zeros(1, dtype=torch.int32, device=DEV)
    hc, pc = pageable.c_struct(), pool.c_struct()
    rc = native.lib().moe_expert_cache_fetch(native.ctypes.byref(hc), native.ctypes.byref(pc), H,
                                             I, native._ptr(fetch), native._ptr(n), 2,
                                             native._stream())
    assert rc == 1 and "pinned" in native.lib().nvfp4_last_error().decode()
