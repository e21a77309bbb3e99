"""GPU parity of the HIP library against the fp64 CPU oracle.

Bit-exact: dequantisation, quantisation codes/scales/global, routing ids,
offsets and permutation.  Tolerance (fp32 outputs): relative Frobenius
error <= 1e-3 and max |error| <= 1e-2 * RMS against the fp64 oracle; bf16
outputs must equal the RNE rounding of the same kernel's fp32 output and sit
within one bf16 ulp of the rounded oracle.  Every call goes through the C ABI.
"""
import sys

import numpy as np
import pytest
import torch

from nvfp4_routed_expert_amd import native, synth, weights
from oracle import nvfp4_oracle as O
from tests.helpers import (LazyOracleExperts, assert_bf16_output, assert_close_f32,
                           check_device_h, rows_by_pair, spread_tokens)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def to_np(t):
    return t.detach().cpu().numpy()


def bf16_np(t):
    return t.detach().cpu().to(torch.float32).numpy()


# ---------------------------------------------------------------------------
# dequantisation and quantisation (bit-exact)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rows,cols", [(1, 32), (37, 96), (256, 512)])
def test_dequantize_bit_exact(rows, cols):
    say("dequantize", rows, cols)
    rng = np.random.default_rng(rows * 1000 + cols)
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, size=(rows, cols // 16), dtype=np.uint8)
    scales.flat[: min(scales.size, 127)] = np.arange(min(scales.size, 127))  # every finite scale
    g = np.float32(0.0371)
    out = native.nvfp4_dequantize(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                                  torch.tensor([g], device=DEV))
    ref = O.dequantize_f32(codes, scales, g)
    assert np.array_equal(to_np(out).view(np.uint32), ref.view(np.uint32))


def _quant_cases():
    rng = np.random.default_rng(0)
    cases = {}
    cases["weights_512x256"] = (synth.weight(512, 256, synth.GATE, 0), torch.float32)
    cases["wide_range"] = ((rng.standard_normal((33, 160)) *
                            np.exp(rng.uniform(-12, 12, (33, 1)))).astype(np.float32), torch.float32)
    # E2M1 half-way points (exact ties when g = 2^-8 is given, see below)
    ties = np.tile(np.array([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.25, -0.75, -1.25, -1.75,
                             -2.5, -3.5, -5, 0], np.float32), (4, 2))
    cases["ties"] = (ties, torch.float32)
    z = rng.standard_normal((8, 64)).astype(np.float32)
    z[2] = 0
    z[5, 16:32] = 0
    z[6, 0:16] *= 1e-9         # a block whose scale underflows
    cases["zeros"] = (z, torch.float32)
    cases["bf16_acts"] = (synth.activations(64, 2048).float().numpy(), torch.bfloat16)
    return cases


@pytest.mark.parametrize("name", list(_quant_cases().keys()))
def test_quantize_bit_exact(name):
    x, dt = _quant_cases()[name]
    say("quantize", name, x.shape, dt)
    xt = torch.from_numpy(x).to(DEV).to(dt)
    codes, scales, g = native.nvfp4_quantize(xt)
    rc, rs, rg = O.quantize(xt.float().cpu().numpy())
    assert to_np(g)[0] == rg
    assert np.array_equal(to_np(scales), rs)
    assert np.array_equal(to_np(codes), rc)
    # given-scale mode: for the tie block g = 2^-8 makes s = 256 and s*g = 1,
    # so every listed element is an exact E2M1 half-way point
    gg = np.float32(2.0 ** -8) if name == "ties" else np.float32(rg * 0.75)
    codes2, scales2, _ = native.nvfp4_quantize(xt, global_scale=torch.tensor([gg], device=DEV))
    rc2, rs2, _ = O.quantize(xt.float().cpu().numpy(), g=gg)
    assert np.array_equal(to_np(scales2), rs2) and np.array_equal(to_np(codes2), rc2)


def test_quantize_strided_rows():
    say("quantize strided")
    x = synth.weight(40, 128, synth.UP, 3)
    big = torch.zeros((40, 192), dtype=torch.float32, device=DEV)
    big[:, :128] = torch.from_numpy(x).to(DEV)
    codes, scales, g = native.nvfp4_quantize(big[:, :128])
    rc, rs, rg = O.quantize(x)
    assert to_np(g)[0] == rg and np.array_equal(to_np(codes), rc) and np.array_equal(to_np(scales), rs)


# ---------------------------------------------------------------------------
# routing (bit-exact integers)
# ---------------------------------------------------------------------------

ROUTE_CASES = [
    ("decode_16x512_k8", 16, 512, 8, None, True),
    ("prefill_512x512_k8_zipf", 512, 512, 8, 1.1, True),
    ("w4a4_2048x128_k8", 2048, 128, 8, None, True),
    ("ragged_37x20_k3", 37, 20, 3, None, True),
    ("no_renorm_19x64_k6", 19, 64, 6, None, False),
    ("k_eq_e_5x7", 5, 7, 7, None, True),
    ("big_e_3x1024_k32", 3, 1024, 32, None, True),
    ("long_9000x64_k2", 9000, 64, 2, None, True),
    ("decode_ties_32x256_k8", 32, 256, 8, None, True),
    ("decode_ties_16x300_k8", 16, 300, 8, None, True),
    ("ragged_2x3_k2", 2, 3, 2, None, False),
    ("one_token_1x512_k8", 1, 512, 8, None, True),
    ("split_ragged_700x301_k5", 700, 301, 5, None, True),     # last expert group short
    ("past_split_lds_300000x2_k1", 300000, 2, 1, None, True),  # bitmaps beyond one workgroup's LDS
]


@pytest.mark.parametrize("case", ROUTE_CASES, ids=[c[0] for c in ROUTE_CASES])
def test_route_topk_parity(case):
    name, T, E, k, zipf, renorm = case
    say("route", name)
    logits = synth.router_logits(T, E, seed=1, zipf_s=zipf)
    if name.startswith("ragged") or "ties" in name:
        logits = np.round(logits * 2) / 2      # plant many ties
    ids, w, off, pairs = native.moe_route_topk(torch.from_numpy(logits).to(DEV), k, renorm)
    rids, rw = O.route_topk(logits, k, renorm)
    roff, rpairs = O.permute(rids, E)
    assert np.array_equal(to_np(ids), rids)
    assert np.array_equal(to_np(off), roff)
    assert np.array_equal(to_np(pairs), rpairs)
    np.testing.assert_allclose(to_np(w), rw, rtol=5e-6, atol=1e-7)


@pytest.mark.parametrize("T", [16, 32])
def test_route_workspace_reused_across_calls(T):
    """One zeroed workspace serves successive decode-sized calls: each call's
    last wavefront resets the counter, and every call is exact."""
    E, k = 512, 8
    say("route workspace reuse", T)
    ws = native.route_workspace(T, E, k, DEV)
    for seed in (3, 4, 5, 6):
        logits = synth.router_logits(T, E, seed=seed)
        if seed == 5:
            logits = np.round(logits)   # ties
        ids, w, off, pairs = native.moe_route_topk(torch.from_numpy(logits).to(DEV), k,
                                                   workspace=ws)
        rids, rw = O.route_topk(logits, k)
        roff, rpairs = O.permute(rids, E)
        assert np.array_equal(to_np(ids), rids)
        assert np.array_equal(to_np(off), roff)
        assert np.array_equal(to_np(pairs), rpairs)
        assert int(to_np(ws[:4].view(torch.int32))[0]) == 0
    # a workspace of unknown contents, made ready by moe_route_workspace_init
    ws.fill_(0xFF)
    native._init_route_workspace(ws)
    logits = synth.router_logits(T, E, seed=7)
    ids, w, off, pairs = native.moe_route_topk(torch.from_numpy(logits).to(DEV), k, workspace=ws)
    rids, _ = O.route_topk(logits, k)
    roff, rpairs = O.permute(rids, E)
    assert np.array_equal(to_np(off), roff) and np.array_equal(to_np(pairs), rpairs)


@pytest.mark.parametrize("T,E,k", [(16, 64, 8), (37, 20, 3), (600, 64, 4), (300000, 2, 1),
                                   (2048, 128, 8)])
def test_permute_drops_ids_outside_the_experts(T, E, k):
    """moe_permute_pairs on ids with dropped pairs (-1 and E): bit-exact with
    the oracle's permutation (kept pairs only, -1 after them), on each of the
    permutation kernels (one workgroup, split by expert, chunked)."""
    say("permute with dropped pairs", T, E, k)
    rng = np.random.default_rng(T + E)
    # distinct experts per token, as routing and slot plans give
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    drop = rng.random((T, k)) < 0.2
    ids[drop] = np.where(rng.random(int(drop.sum())) < 0.5, -1, E)
    off, pairs = native.moe_permute_pairs(torch.from_numpy(ids).to(DEV), E)
    roff, rpairs = O.permute(ids, E)
    assert np.array_equal(to_np(off), roff)
    assert np.array_equal(to_np(pairs), rpairs)


# ---------------------------------------------------------------------------
# BF16 router + top-k
# ---------------------------------------------------------------------------

# tiles: T < 64 one 16x16 subtile per wavefront with K split into up to 32
# parts; T < 256 32x32; larger 64x64 (K split into up to 8 parts)
@pytest.mark.parametrize("T,H,E,k,zipf,renorm", [
    (16, 2048, 512, 8, None, True),      # the decode workload's router
    (37, 96, 20, 3, None, True),         # ragged tiles, H % 64 == 32
    (1, 32, 1, 1, None, True),           # one token, one expert
    (300, 256, 64, 6, 1.1, False),       # 32 x 32 tiles, bias, full softmax
    (1024, 512, 128, 8, None, True),     # 64 x 64 tiles
    (512, 2048, 512, 8, 1.1, True),      # the 512-token chunk's router (Zipf bias)
    (40, 160, 1024, 32, None, True),     # the largest E and k
])
def test_router_topk_parity(T, H, E, k, zipf, renorm):
    say("router", T, H, E, k, zipf, renorm)
    x = synth.activations(T, H, seed=2)
    R = synth.router_matrix(E, H, seed=2)
    b = None if zipf is None else synth.zipf_bias(E, zipf)
    bd = None if b is None else torch.from_numpy(b).to(DEV)
    ids, w, off, pairs, lg = native.moe_router_topk(x.to(DEV), R.to(DEV), k, renorm, bias=bd,
                                                    want_logits=True)
    lg = to_np(lg)
    xf, rf = x.float().numpy().astype(np.float64), R.float().numpy().astype(np.float64)
    ref = O.router_logits(xf, rf, b)
    # fp32 sums of exact products: |err| <= H u sum_h |x_h r_h| (u = 2^-24),
    # plus one rounding of the bias add
    bound = H * 2.0 ** -24 * (np.abs(xf) @ np.abs(rf).T) + 2.0 ** -24 * np.abs(ref)
    assert np.all(np.abs(lg - ref) <= bound), float(np.max(np.abs(lg - ref) - bound))
    # the routing decision, taken on the same fp32 logits: exact
    rids, rw = O.route_topk(lg, k, renorm)
    roff, rpairs = O.permute(rids, E)
    assert np.array_equal(to_np(ids), rids)
    assert np.array_equal(to_np(off), roff)
    assert np.array_equal(to_np(pairs), rpairs)
    np.testing.assert_allclose(to_np(w), rw, rtol=5e-6, atol=1e-7)
    # and the fp64 oracle's own choice for every token whose top k + 1 fp64
    # logits lie further apart than twice the token's largest logit error
    # (then both orders agree)
    ids64, _ = O.route_topk(ref, k, renorm)
    srt = -np.sort(-ref, axis=1)[:, :min(k + 1, E)]
    err = np.abs(lg - ref).max(axis=1, keepdims=True)
    clear = np.all(np.diff(-srt, axis=1) > 2 * err, axis=1)
    assert clear.mean() > 0.9
    assert np.array_equal(to_np(ids)[clear], ids64[clear])
    # no logits requested: same routing; a second call is bit-identical
    ids2, w2, off2, pairs2, _ = native.moe_router_topk(x.to(DEV), R.to(DEV), k, renorm, bias=bd)
    assert torch.equal(ids, ids2) and torch.equal(w, w2) and torch.equal(pairs, pairs2)


# ---------------------------------------------------------------------------
# BF16 shared expert
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,H,I", [
    (16, 2048, 512),      # beside the decode workload (one-subtile tiles, K split)
    (37, 96, 160),        # ragged tiles, H and I % 64 == 32
    (1, 32, 32),          # one token, one K step
    (300, 256, 512),      # 32 x 32 tiles
    (512, 2048, 512),     # beside the 512-token chunk
])
def test_shared_expert_parity(T, H, I):
    say("shared expert", T, H, I)
    x = synth.activations(T, H, seed=4)
    wg, wu, wd = synth.shared_expert_weights(H, I, seed=4)
    dx, dg, du, dd = (t.to(DEV) for t in (x, wg, wu, wd))
    y32 = native.moe_shared_expert_ffn(dx, dg, du, dd, out_dtype=torch.float32)
    ref = O.shared_expert(x.float().numpy(), wg.float().numpy(), wu.float().numpy(),
                          wd.float().numpy())
    assert_close_f32(to_np(y32), ref, "shared expert")
    # bf16 output: the same sums, rounded once
    yb = native.moe_shared_expert_ffn(dx, dg, du, dd, out_dtype=torch.bfloat16)
    assert_bf16_output(bf16_np(yb), to_np(y32), ref, "shared expert bf16")
    # accumulate into a given output (the routed result): fl32(y_in + s), then
    # one rounding to y's type
    y_in = torch.from_numpy(np.random.default_rng(T).standard_normal((T, H)).astype(np.float32))
    ya = y_in.to(DEV).clone()
    native.moe_shared_expert_ffn(dx, dg, du, dd, y=ya, accumulate=True)
    assert np.array_equal(to_np(ya), (y_in.numpy() + to_np(y32)).astype(np.float32))
    yab = y_in.to(torch.bfloat16).to(DEV)
    want = O.bf16_rne((bf16_np(yab).astype(np.float32) + to_np(y32).astype(np.float32))
                      .astype(np.float32))
    native.moe_shared_expert_ffn(dx, dg, du, dd, y=yab, accumulate=True)
    assert np.array_equal(bf16_np(yab), want)
    # deterministic
    assert torch.equal(native.moe_shared_expert_ffn(dx, dg, du, dd, out_dtype=torch.float32), y32)


# ---------------------------------------------------------------------------
# dense NVFP4 linear
# ---------------------------------------------------------------------------

def _linear_inputs(M, K, N, seed=0):
    x = synth.activations(M, K, seed)
    wf = synth.weight(N, K, synth.GATE, 0, seed)
    return x, wf


# M <= 16 with K in {256, 512, 1024, 2048..8192} takes the row-streaming
# kernel (N need not fill its 8/16/32/64-row items); the rest the MFMA kernel
@pytest.mark.parametrize("M,K,N", [(4, 256, 512), (1, 32, 16), (5, 96, 40), (17, 160, 48),
                                   (33, 256, 64), (130, 384, 96), (3, 2048, 40), (16, 5120, 24),
                                   (2, 1024, 100), (7, 512, 64), (1, 8192, 13)])
def test_linear_w4a16(M, K, N):
    say("linear w4a16", M, K, N)
    x, wf = _linear_inputs(M, K, N)
    codes, scales, g = native.nvfp4_quantize(torch.from_numpy(wf).to(DEV))
    rc, rs, rg = O.quantize(wf)
    assert np.array_equal(to_np(codes), rc)
    xd = x.to(DEV)
    y32, _ = native.nvfp4_linear(xd, codes, scales, g, out_dtype=torch.float32)
    yb, _ = native.nvfp4_linear(xd, codes, scales, g, out_dtype=torch.bfloat16)
    ref, _ = O.linear(x.float().numpy(), rc, rs, rg)
    assert_close_f32(to_np(y32), ref, "linear f32")
    assert_bf16_output(bf16_np(yb), to_np(y32), ref, "linear bf16")


@pytest.mark.parametrize("given", [False, True])
def test_linear_w4a4(given):
    M, K, N = 24, 256, 128
    say("linear w4a4 given" if given else "linear w4a4 compute")
    x, wf = _linear_inputs(M, K, N, seed=2)
    codes, scales, g = native.nvfp4_quantize(torch.from_numpy(wf).to(DEV))
    rc, rs, rg = O.quantize(wf)
    xn = x.float().numpy()
    gx_ref = O.tensor_global(xn) * (np.float32(1.5) if given else np.float32(1))
    ag = torch.tensor([gx_ref], device=DEV) if given else None
    y32, gx = native.nvfp4_linear(x.to(DEV), codes, scales, g, act=native.W4A4, act_global=ag,
                                  out_dtype=torch.float32)
    ref, rgx = O.linear(xn, rc, rs, rg, act_quant=True, act_global=gx_ref if given else None)
    assert to_np(gx)[0] == rgx
    assert_close_f32(to_np(y32), ref, "linear w4a4")


# ---------------------------------------------------------------------------
# routed-expert FFN
# ---------------------------------------------------------------------------

_ORACLE_CACHE = {}


def oracle_experts(E, H, I, need, seed):
    key = (E, H, I, seed, tuple(int(e) for e in need))
    if key not in _ORACLE_CACHE:
        _ORACLE_CACHE.clear()
        _ORACLE_CACHE[key] = LazyOracleExperts(E, H, I, need, seed)
    return _ORACLE_CACHE[key]


def _moe_run(T, H, I, E, k, act=native.W4A16, zipf=None, seed=0, tokens=None,
             given_globals=None, out_dtype=torch.float32, experts_needed=None):
    x = synth.activations(T, H, seed)
    logits = synth.router_logits(T, E, seed, zipf_s=zipf)
    rids, rw = O.route_topk(logits, k)
    sel = rids if tokens is None else rids[tokens]
    need = np.unique(sel) if experts_needed is None else experts_needed
    w_gpu = weights.synthetic_experts(E, H, I, seed, DEV, experts=np.unique(rids))
    ids, wts, off, pairs = native.moe_route_topk(torch.from_numpy(logits).to(DEV), k)
    ag = None if given_globals is None else torch.tensor(given_globals, dtype=torch.float32,
                                                         device=DEV)
    y, g_out = native.moe_grouped_nvfp4_ffn(x.to(DEV), w_gpu, ids, wts, off, pairs, k, act=act,
                                            act_globals=ag, out_dtype=out_dtype)
    w_ref = oracle_experts(E, H, I, need, seed)
    return x, rids, rw, y, g_out, w_ref, (ids, wts, off, pairs, w_gpu)


# decode-shaped cases (at most 16 pairs per expert on average) take the
# row-streaming kernels when H and I are 256, 512, 1024 or 2048..8192; the
# others take the MFMA kernels
@pytest.mark.parametrize("T,H,I,E,k", [(37, 256, 160, 8, 2), (1, 64, 32, 4, 1), (12, 128, 96, 6, 6),
                                       (40, 512, 256, 16, 4), (24, 2048, 1024, 32, 4),
                                       (9, 5120, 512, 16, 2), (30, 4096, 256, 24, 6),
                                       (3, 1024, 2048, 64, 8),
                                       # H = 2048 takes the fused decode kernel: 1 and 9 slices of I,
                                       # one token with one slot, the largest decode batch (256 pairs)
                                       (16, 2048, 256, 64, 8), (5, 2048, 2304, 16, 3),
                                       (1, 2048, 512, 512, 1), (32, 2048, 512, 512, 8)])
def test_moe_ffn_w4a16_small(T, H, I, E, k):
    say("moe w4a16 small", T, H, I, E, k)
    import bench
    if H == 2048:   # the cases labelled fused do take the fused decode kernel
        assert bench.gate_up_kernel(T, H, I, E, k, "w4a16") == "row_ffn_kernel"
    x, rids, rw, y, _, w_ref, st = _moe_run(T, H, I, E, k)
    ref, _ = O.moe_ffn(x.float().numpy(), rids, rw, w_ref)
    assert_close_f32(to_np(y), ref, "moe w4a16")
    # bf16 output: same kernels, rounded once
    ids, wts, off, pairs, w_gpu = st
    yb, _ = native.moe_grouped_nvfp4_ffn(x.to(DEV), w_gpu, ids, wts, off, pairs, k,
                                         out_dtype=torch.bfloat16)
    assert_bf16_output(bf16_np(yb), to_np(y), ref, "moe bf16")
    # deterministic: a second run is bit-identical
    y2, _ = native.moe_grouped_nvfp4_ffn(x.to(DEV), w_gpu, ids, wts, off, pairs, k,
                                         out_dtype=torch.float32)
    assert torch.equal(y, y2)


# prefill-shaped cases (more than 256 pairs) take the grouped GEMM over
# m-blocks of 128 rows; H or I not a multiple of 64 takes its fallback kernel.
# zipf: one expert takes most tokens (several m-blocks, a ragged last one).
@pytest.mark.parametrize("T,H,I,E,k,zipf", [(80, 256, 192, 8, 4, None), (129, 128, 128, 3, 2, None),
                                            (300, 512, 256, 16, 2, None), (70, 320, 96, 5, 4, None),
                                            (333, 256, 128, 32, 2, 3.0), (600, 192, 64, 64, 1, 2.0)])
def test_moe_ffn_w4a16_tiles(T, H, I, E, k, zipf):
    say("moe w4a16 tiles", T, H, I, E, k, zipf)
    x, rids, rw, y, _, w_ref, st = _moe_run(T, H, I, E, k, zipf=zipf)
    counts = np.bincount(rids.ravel(), minlength=E)
    ref, _ = O.moe_ffn(x.float().numpy(), rids, rw, w_ref)
    assert_close_f32(to_np(y), ref, f"moe tiles (max rows per expert {counts.max()})")
    ids, wts, off, pairs, w_gpu = st
    yb, _ = native.moe_grouped_nvfp4_ffn(x.to(DEV), w_gpu, ids, wts, off, pairs, k,
                                         out_dtype=torch.bfloat16)
    assert_bf16_output(bf16_np(yb), to_np(y), ref, "moe tiles bf16")
    y2, _ = native.moe_grouped_nvfp4_ffn(x.to(DEV), w_gpu, ids, wts, off, pairs, k,
                                         out_dtype=torch.float32)
    assert torch.equal(y, y2)


# W4A16 grouped-GEMM batches with skewed and flat routing: experts with a few
# rows beside experts with several m-blocks, every expert with a few rows,
# every expert with many
@pytest.mark.parametrize("T,H,I,E,k,zipf", [(400, 256, 256, 64, 4, 1.1),
                                            (512, 512, 512, 128, 8, 1.1),   # the chunk's shape, smaller
                                            (300, 256, 512, 256, 1, None),
                                            (700, 1024, 256, 8, 2, None)])
def test_moe_ffn_w4a16_skewed_batches(T, H, I, E, k, zipf):
    say("moe w4a16 skewed", T, H, I, E, k, zipf)
    x, rids, rw, y, _, w_ref, st = _moe_run(T, H, I, E, k, zipf=zipf)
    counts = np.bincount(rids.ravel(), minlength=E)
    say("experts with 1..8 rows", int(((counts > 0) & (counts <= 8)).sum()),
        "with more", int((counts > 8).sum()))
    ref, _ = O.moe_ffn(x.float().numpy(), rids, rw, w_ref)
    assert_close_f32(to_np(y), ref, "moe skewed")
    ids, wts, off, pairs, w_gpu = st
    y2, _ = native.moe_grouped_nvfp4_ffn(x.to(DEV), w_gpu, ids, wts, off, pairs, k,
                                         out_dtype=torch.float32)
    assert torch.equal(y, y2)


@pytest.mark.parametrize("T,I,E,k", [(16, 512, 512, 8), (5, 2304, 16, 3), (32, 512, 512, 8)])
def test_fused_decode_in_pair_order(T, I, E, k):
    """The fused decode path given no permutation (expert_offsets and
    sorted_pairs NULL) reads the pairs in pair order: bit-identical to the
    call with the permutation, also with dropped slots (ids -1 and E); the
    top-k alone (moe_route_topk without its permutation outputs) gives the
    same ids and weights; NULL permutation outputs are refused off that
    path."""
    import bench
    H = 2048
    assert bench.gate_up_kernel(T, H, I, E, k, "w4a16") == "row_ffn_kernel"
    say("fused decode pair order", T, H, I, E, k)
    x = synth.activations(T, H, 4).to(DEV)
    logits = torch.from_numpy(synth.router_logits(T, E, 4)).to(DEV)
    ids, wts, off, pairs = native.moe_route_topk(logits, k)
    ids2, wts2, off2, pairs2 = native.moe_route_topk(logits, k, permute=False)
    assert off2 is None and pairs2 is None
    assert torch.equal(ids, ids2) and torch.equal(wts, wts2)
    w = weights.synthetic_experts(E, H, I, 4, DEV, experts=np.unique(to_np(ids)))
    for ids_c in (ids, ids.clone().index_fill_(1, torch.tensor([0], device=DEV), -1)):
        if ids_c is not ids:
            ids_c[1, :] = -1
            ids_c[2, k - 1] = E
        off_c, pairs_c = native.moe_permute_pairs(ids_c, E)
        for dt in (torch.float32, torch.bfloat16):
            y_ref, _ = native.moe_grouped_nvfp4_ffn(x, w, ids_c, wts, off_c, pairs_c, k,
                                                    out_dtype=dt)
            y_po, _ = native.moe_grouped_nvfp4_ffn(x, w, ids_c, wts, None, None, k, out_dtype=dt)
            torch.cuda.synchronize()
            assert torch.equal(y_po, y_ref), (dt, ids_c is ids)
    with pytest.raises(native.NVFP4Error):   # not the fused decode path
        native.moe_grouped_nvfp4_ffn(x, w, ids, wts, None, None, k, act=native.W4A4)


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.parametrize("T,I,E,k,renorm,ties", [
    (16, 512, 512, 8, True, False),    # the decode workload
    (16, 512, 512, 8, True, True),     # planted ties in the logits
    (5, 2304, 16, 3, False, False),    # nine slices, softmax over all experts
    (32, 512, 512, 8, True, False),    # 256 pairs: four permutation slots
    (1, 256, 8, 2, True, False),       # one token, one slice
])
def test_route_ffn_decode_bit_identical(T, I, E, k, renorm, ties):
    """moe_route_ffn_decode (each FFN workgroup routes its own token; the
    combine launch makes the permutation) equals moe_route_topk followed by
    moe_grouped_nvfp4_ffn bit for bit in all five outputs, and its ids equal
    the oracle's top-k; the decode routing's workgroup-wide top-k equals the
    per-lane merge network's bit for bit."""
    H = 2048
    say("route + ffn decode", T, H, I, E, k, renorm, ties)
    x = synth.activations(T, H, 5).to(DEV)
    lg = synth.router_logits(T, E, 5)
    if ties:
        lg = np.round(lg * 2) / 2
    logits = torch.from_numpy(lg).to(DEV)
    ids, wts, off, pairs = native.moe_route_topk(logits, k, renorm)
    # the top-k alone runs the per-lane merge network instead of the
    # workgroup-wide one: the same ids and weights, bit for bit
    ids1, wts1, _, _ = native.moe_route_topk(logits, k, renorm, permute=False)
    assert torch.equal(ids1, ids) and torch.equal(_bits(wts1), _bits(wts))
    rids, _ = O.route_topk(lg, k, renorm)
    w = weights.synthetic_experts(E, H, I, 5, DEV, experts=np.unique(to_np(ids)))
    for dt in (torch.bfloat16, torch.float32):
        y_ref, _ = native.moe_grouped_nvfp4_ffn(x, w, ids, wts, off, pairs, k, out_dtype=dt)
        y, (ids2, wts2, off2, pairs2) = native.moe_route_ffn_decode(logits, x, w, k, renorm,
                                                                    out_dtype=dt)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(ids2), rids)
        assert torch.equal(ids2, ids) and torch.equal(_bits(wts2), _bits(wts))
        assert torch.equal(off2, off) and torch.equal(pairs2, pairs)
        assert torch.equal(_bits(y), _bits(y_ref)), dt
    with pytest.raises(native.NVFP4Error):   # H = 2048 only
        native.moe_route_ffn_decode(logits, synth.activations(T, 1024, 5).to(DEV), w, k)


def test_moe_ffn_in_a_graph():
    """The grouped-GEMM FFN captured into a graph: every replay (with eager
    calls between them) equals the eager result bit for bit."""
    T, H, I, E, k = 400, 256, 256, 64, 4
    say("moe ffn graph", T, H, I, E, k)
    x, rids, rw, y, _, w_ref, st = _moe_run(T, H, I, E, k, zipf=1.1)
    ids, wts, off, pairs, w_gpu = st
    xd = x.to(DEV)
    ws = torch.empty(native.ffn_workspace_bytes(T, H, I, E, k), dtype=torch.uint8, device=DEV)
    out = torch.empty((T, H), dtype=torch.float32, device=DEV)

    def call():
        native.moe_grouped_nvfp4_ffn(xd, w_gpu, ids, wts, off, pairs, k, out_dtype=torch.float32,
                                     workspace=ws, out=out)
    call()
    torch.cuda.synchronize()
    eager = out.clone()
    assert torch.equal(eager, y)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        y2, _ = native.moe_grouped_nvfp4_ffn(xd, w_gpu, ids, wts, off, pairs, k,
                                             out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(y2, eager)


def test_route_ffn_decode_in_a_graph():
    """moe_route_ffn_decode (routing inside the fused decode launch, the
    permutation beside the combine) captured into a graph: every replay,
    with eager calls between them, writes the eager call's five outputs bit
    for bit (all outputs are cleared before each replay)."""
    T, H, I, E, k = 16, 2048, 512, 512, 8
    say("route + ffn decode graph", T, H, I, E, k)
    x = synth.activations(T, H, 6).to(DEV)
    logits = torch.from_numpy(synth.router_logits(T, E, 6)).to(DEV)
    ids0, _, _, _ = native.moe_route_topk(logits, k)
    w = weights.synthetic_experts(E, H, I, 6, DEV, experts=np.unique(to_np(ids0)))
    outs = (torch.empty((T, k), dtype=torch.int32, device=DEV),
            torch.empty((T, k), dtype=torch.float32, device=DEV),
            torch.empty(E + 1, dtype=torch.int32, device=DEV),
            torch.empty(T * k, dtype=torch.int32, device=DEV))
    y = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(native.lib().moe_route_ffn_decode_workspace_size(T, H, I, E, k),
                     dtype=torch.uint8, device=DEV)

    def call():
        native.moe_route_ffn_decode(logits, x, w, k, route_out=outs, out=y, workspace=ws)
    call()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs] + [y.clone()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(3):
        for t in list(outs) + [y]:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = list(outs) + [y]
        assert all(torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a, b.view(
            torch.int16) if b.dtype == torch.bfloat16 else b) for a, b in zip(got, eager)), i
        y2, _ = native.moe_route_ffn_decode(logits, x, w, k)   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y2.view(torch.int16), eager[4].view(torch.int16))


def _w4a4_device_h_check(x, rids, rw, w_ref, st, y, g_out, T, H, I, E, k, tokens=None,
                         given=False, ws=None):
    """Reads the device's bf16 h and W4A4 operand from the FFN's workspace
    and runs the several-results-correct check (tests.helpers.check_device_h)
    on the sampled tokens; also checks g_x, and g_h against the device's own h
    (bit-exact).  Returns (flips, flagged, checked)."""
    ids, wts, off, pairs, w_gpu = st
    P = T * k
    hb, hq = native.ffn_debug_h(ws, T, H, I, E, k, native.W4A4, given)
    assert hb is not None, "this call keeps no bf16 h in its workspace"
    sp = to_np(pairs)
    h_pairs = rows_by_pair(to_np(hb), sp, P)
    hq_pairs = None if hq is None else rows_by_pair(to_np(hq), sp, P)
    xf = x.float().numpy()
    g_x, g_h = to_np(g_out)[0], to_np(g_out)[1]
    assert g_x == O.tensor_global(xf)
    kept_rows = h_pairs[~np.isnan(h_pairs[:, 0])]
    if not given:   # the online h scale is the device h's own
        assert g_h == O.tensor_global(kept_rows.astype(np.float32))
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    fl = check_device_h(xf, rids, rw, w_ref, h_pairs, hq_pairs, g_x, g_h, tokens, True,
                        to_np(y)[tokens], f"w4a4 T={T} H={H} I={I} E={E} k={k}")
    say("h flips / flagged / checked", *fl)
    return fl


def _ffn_ws(T, H, I, E, k, act):
    return torch.empty(native.ffn_workspace_bytes(T, H, I, E, k, act), dtype=torch.uint8,
                       device=DEV)


@pytest.mark.parametrize("T,H,I,E,k", [(37, 256, 160, 8, 2), (64, 512, 256, 16, 4),
                                       (96, 256, 128, 8, 4), (300, 256, 512, 16, 2)])
def test_moe_ffn_w4a4_small(T, H, I, E, k):
    """W4A4 with online globals (GEMV and tiled paths): g_x bit-exact, the
    device's h a valid rounding of the fp64 h everywhere, its NVFP4 codes
    and g_h exact for that h, and the output within tolerance of the oracle
    run downstream from it."""
    say("moe w4a4 small", T, H, I, E, k)
    x, rids, rw, _, _, w_ref, st = _moe_run(T, H, I, E, k, act=native.W4A4)
    ids, wts, off, pairs, w_gpu = st
    ws = _ffn_ws(T, H, I, E, k, native.W4A4)
    y, g_out = native.moe_grouped_nvfp4_ffn(x.to(DEV), w_gpu, ids, wts, off, pairs, k,
                                            act=native.W4A4, out_dtype=torch.float32,
                                            workspace=ws)
    torch.cuda.synchronize()
    _w4a4_device_h_check(x, rids, rw, w_ref, st, y, g_out, T, H, I, E, k, ws=ws)
    # the fp64 oracle run on its own h stays within the bound as well
    ref, info = O.moe_ffn(x.float().numpy(), rids, rw, w_ref, act_quant=True)
    assert to_np(g_out)[0] == info["g_x"]
    assert abs(to_np(g_out)[1] / info["g_h"] - 1) <= 2 ** -7
    # with the oracle's own globals given, the two runs agree as well
    ids, wts, off, pairs, w_gpu = st
    yg, _ = native.moe_grouped_nvfp4_ffn(
        x.to(DEV), w_gpu, ids, wts, off, pairs, k, act=native.W4A4,
        act_globals=torch.tensor([info["g_x"], info["g_h"]], device=DEV), out_dtype=torch.float32)
    refg, _ = O.moe_ffn(x.float().numpy(), rids, rw, w_ref, act_quant=True,
                        act_globals=(info["g_x"], info["g_h"]))
    assert_close_f32(to_np(yg), refg, "moe w4a4 given")


def test_moe_single_expert_is_dense_mlp():
    say("moe E=1 k=1")
    T, H, I = 9, 256, 192
    x, rids, rw, y, _, w_ref, _ = _moe_run(T, H, I, 1, 1)
    ref = O.dense_mlp(x.float().numpy(), (w_ref.gate_codes[0], w_ref.gate_scales[0], w_ref.gate_global[0]),
                      (w_ref.up_codes[0], w_ref.up_scales[0], w_ref.up_global[0]),
                      (w_ref.down_codes[0], w_ref.down_scales[0], w_ref.down_global[0]))
    assert_close_f32(to_np(y), ref, "dense mlp via moe")


@pytest.mark.parametrize("H,I", [(1024, 256), (2048, 4352), (3072, 2112), (5120, 1024),
                                 (4096, 2048), (1024, 31744)])
def test_one_row_dense_mlp(H, I):
    """One row of a dense MLP (one expert, one slot) takes the gate/up kernel
    that deals I out evenly as whole 16-column blocks and the down kernel
    that deals the H output rows out evenly and writes y: against the oracle's dense MLP in fp32 and as its bf16
    rounding.  Cases: 16 to 132 workgroups of one block (132: a ragged last
    XCD range), 256 workgroups of one or two blocks (4352) and of up to
    eight (31744, the most a workgroup takes, and the longest h the down
    kernel stages in LDS), a 1024-element piece in the x row for odd
    H / 1024, and K slices of the down rows cut short (I % 2048 = 256, 64,
    1024)."""
    import bench
    assert bench.gate_up_kernel(1, H, I, 1, 1, "w4a16") == "row_mlp_gate_up_kernel"
    say("one-row dense mlp", H, I)
    x, rids, rw, y, _, w_ref, st = _moe_run(1, H, I, 1, 1, seed=H + I)
    ref = O.dense_mlp(x.float().numpy(), (w_ref.gate_codes[0], w_ref.gate_scales[0], w_ref.gate_global[0]),
                      (w_ref.up_codes[0], w_ref.up_scales[0], w_ref.up_global[0]),
                      (w_ref.down_codes[0], w_ref.down_scales[0], w_ref.down_global[0]))
    assert_close_f32(to_np(y), ref, "one-row dense mlp")
    ids, wts, off, pairs, w_gpu = st
    yb, _ = native.moe_grouped_nvfp4_ffn(x.to(DEV), w_gpu, ids, wts, off, pairs, 1,
                                         out_dtype=torch.bfloat16)
    assert_bf16_output(to_np(yb.float()), to_np(y), ref, "one-row dense mlp (bf16)")


def test_one_row_dense_mlp_dropped_and_repeated():
    """The one-row path with a dropped id writes zeros (y filled with NaN
    first); repeated calls through one workspace, and a captured graph's
    replays with eager calls between them, give the eager result bit for
    bit."""
    H, I = 2048, 2112
    say("one-row dense mlp dropped / graph", H, I)
    x = synth.activations(1, H, 5).to(DEV)
    w_gpu = weights.synthetic_experts(1, H, I, 5, DEV)
    wts = torch.ones((1, 1), dtype=torch.float32, device=DEV)
    ws = torch.empty(native.ffn_workspace_bytes(1, H, I, 1, 1), dtype=torch.uint8, device=DEV)
    for bad in (-1, 1):
        ids = torch.full((1, 1), bad, dtype=torch.int32, device=DEV)
        off, pairs = native.moe_permute_pairs(ids, 1)
        y = torch.full((1, H), float("nan"), dtype=torch.float32, device=DEV)
        native.moe_grouped_nvfp4_ffn(x, w_gpu, ids, wts, off, pairs, 1, out_dtype=torch.float32,
                                     workspace=ws, out=y)
        torch.cuda.synchronize()
        assert torch.all(y == 0.0), bad
    ids = torch.zeros((1, 1), dtype=torch.int32, device=DEV)
    off, pairs = native.moe_permute_pairs(ids, 1)
    out = torch.empty((1, H), dtype=torch.float32, device=DEV)

    def call():
        native.moe_grouped_nvfp4_ffn(x, w_gpu, ids, wts, off, pairs, 1, out_dtype=torch.float32,
                                     workspace=ws, out=out)
    call()
    torch.cuda.synchronize()
    eager = out.clone()
    assert torch.isfinite(eager).all()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(out, eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        call()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


# ---- the full-size workloads, checked on sampled tokens ----------------------------

def test_moe_decode_full_size():
    """The routed decode workload at full size, every token, fp32 and bf16
    outputs (the benchmarked launch configuration)."""
    wl = synth.MOE_DECODE
    say("moe decode full size", wl)
    x, rids, rw, y, _, w_ref, st = _moe_run(wl.T, wl.H, wl.I, wl.E, wl.k)
    ref, _ = O.moe_ffn(x.float().numpy(), rids, rw, w_ref)
    assert_close_f32(to_np(y), ref, "moe decode")
    ids, wts, off, pairs, w_gpu = st
    yb, _ = native.moe_grouped_nvfp4_ffn(x.to(DEV), w_gpu, ids, wts, off, pairs, wl.k,
                                         out_dtype=torch.bfloat16)
    assert_bf16_output(bf16_np(yb), to_np(y), ref, "moe decode bf16")


def _block_covering_tokens(rids, e, bm, extra):
    """Tokens of expert e that land in every bm-row block of its expert-sorted
    rows (first and last row of each block), plus `extra` other tokens."""
    rows = np.nonzero((np.asarray(rids) == e).any(axis=1))[0]   # ascending: the sorted order
    pick = set()
    for b0 in range(0, len(rows), bm):
        pick.add(int(rows[b0]))
        pick.add(int(rows[min(b0 + bm, len(rows)) - 1]))
    pick |= set(int(t) for t in extra)
    return sorted(pick)


def test_moe_prefill_full_size_sampled():
    """The 512-token chunk (Zipf-skewed routing) at full size: tokens at the
    first and last row of every 64-row block of the heaviest expert (gate/up
    block size) and of every 32-row block (down), plus tokens spread over the
    chunk: at least 32 tokens."""
    wl = synth.MOE_PREFILL
    say("moe prefill full size", wl)
    logits = synth.router_logits(wl.T, wl.E, 0, zipf_s=wl.zipf_s)
    rids, _ = O.route_topk(logits, wl.k)
    heavy = int(np.bincount(rids.ravel(), minlength=wl.E).argmax())
    tokens = _block_covering_tokens(rids, heavy, 32, range(0, wl.T, 37))
    assert len(tokens) >= 32
    x, rids, rw, y, _, w_ref, st = _moe_run(wl.T, wl.H, wl.I, wl.E, wl.k, zipf=wl.zipf_s,
                                            tokens=tokens)
    off = to_np(st[2])
    counts = np.diff(off)
    say("active experts", int((counts > 0).sum()), "max tokens per expert", int(counts.max()),
        "tokens checked", len(tokens))
    ref, _ = O.moe_ffn(x.float().numpy(), rids, rw, w_ref, tokens=tokens)
    assert_close_f32(to_np(y)[tokens], ref, "moe prefill")


def _fused_vs_separate(T, H, I, E, k, gh, seed, tokens=None):
    """W4A4 with given globals, h quantised in the gate/up epilogue and in a
    pass of its own: the two outputs and the two h operands are bit-identical,
    and the separate pass's bf16 h passes the several-results-correct check
    (valid roundings of the fp64 h; codes exact for it; output to tolerance
    downstream from it)."""
    x = synth.activations(T, H, seed=seed)
    gx = O.tensor_global(x.float().numpy())
    _, rids, rw, _, _, w_ref, st = _moe_run(T, H, I, E, k, act=native.W4A4, seed=seed,
                                            given_globals=[gx, np.float32(gh)], tokens=tokens)
    ids, wts, off, pairs, w_gpu = st
    ag = torch.tensor([gx, np.float32(gh)], dtype=torch.float32, device=DEV)
    ws_f, ws_s = _ffn_ws(T, H, I, E, k, native.W4A4), _ffn_ws(T, H, I, E, k, native.W4A4)
    y, _ = native.moe_grouped_nvfp4_ffn(x.to(DEV), w_gpu, ids, wts, off, pairs, k,
                                        act=native.W4A4, act_globals=ag,
                                        out_dtype=torch.float32, workspace=ws_f)
    torch.cuda.synchronize()
    _, hq_f = native.ffn_debug_h(ws_f, T, H, I, E, k, native.W4A4, given=True)
    native.set_ffn_separate_h_quant(True)
    try:
        ys, _ = native.moe_grouped_nvfp4_ffn(x.to(DEV), w_gpu, ids, wts, off, pairs, k,
                                             act=native.W4A4, act_globals=ag,
                                             out_dtype=torch.float32, workspace=ws_s)
        torch.cuda.synchronize()
        hb_s, hq_s = native.ffn_debug_h(ws_s, T, H, I, E, k, native.W4A4, given=True)
    finally:
        native.set_ffn_separate_h_quant(False)
    assert torch.equal(y, ys), "fused and separate h quantisation differ"
    kept = to_np(pairs) >= 0
    assert np.array_equal(to_np(hq_f)[kept], to_np(hq_s)[kept]), "h operands differ"
    P = T * k
    sp = to_np(pairs)
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    fl = check_device_h(x.float().numpy(), rids, rw, w_ref, rows_by_pair(to_np(hb_s), sp, P),
                        rows_by_pair(to_np(hq_s), sp, P), gx, np.float32(gh), tok, True,
                        to_np(y)[tok], f"w4a4 given g_h={gh}")
    say("h flips / flagged / checked", *fl)
    return fl


# g_h: 0.05/2688 saturates nearly every block scale at 448; 1.1484375/2688 is
# this input's own h maximum over 2688 (a static scale calibrated on it);
# 2/2688 leaves every block scale small
@pytest.mark.parametrize("gh", [0.05 / 2688, 1.1484375 / 2688, 2.0 / 2688])
def test_moe_ffn_w4a4_h_quantised_in_gate_up_epilogue_matches_separate_pass(gh):
    """Given globals on the four-wave tiled path without a K split: the
    gate/up epilogue quantises h (16-column blocks reduced across lanes).
    Its output and operand are bit-identical to quantising the same bf16 h
    in a pass of its own, and that h is a valid rounding of the fp64 h."""
    T, H, I, E, k = 1024, 256, 2048, 16, 2
    say("moe w4a4 fused h quant", T, H, I, E, k, gh)
    _fused_vs_separate(T, H, I, E, k, gh, seed=3)


# H = 128 is two 64-wide K chunks, which the tiled GEMM never splits, so these
# run the one-wave tiles with the fused epilogue (ragged m-blocks included)
@pytest.mark.parametrize("T,H,I,E,k", [(96, 128, 512, 4, 2), (300, 128, 256, 16, 2)])
@pytest.mark.parametrize("gh", [0.5 / 2688, 2.0 / 2688])
def test_moe_ffn_w4a4_fused_h_quant_one_wave_tiles(T, H, I, E, k, gh):
    say("moe w4a4 fused h quant one-wave", T, H, I, E, k, gh)
    _fused_vs_separate(T, H, I, E, k, gh, seed=5)


@pytest.mark.timeout(900)
def test_moe_w4a4_full_size_online_globals():
    """The W4A4 prefill workload at full size, in the mode it is benchmarked
    (online x and h globals): g_x bit-exact; g_h exact for the device's own
    h; on 16 tokens spread over the batch, every h value a valid rounding of
    the fp64 h, its NVFP4 codes exact, and the outputs within tolerance of
    the oracle downstream from it.  Then the same step with that g_h given as
    a static scale (the run's own amax(h)/2688, the fused epilogue) gives the
    identical output and h operand."""
    wl = synth.MOE_PREFILL_W4A4
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    say("moe w4a4 full size online", wl)
    x = synth.activations(T, H)
    logits = synth.router_logits(T, E)
    rids, rw = O.route_topk(logits, k)
    tokens = spread_tokens(rids, 16)
    need = np.unique(rids[tokens])
    say("tokens", tokens, "experts for the oracle", len(need))
    import concurrent.futures
    pool = concurrent.futures.ThreadPoolExecutor(max_workers=1)
    fut = pool.submit(LazyOracleExperts, E, H, I, need, 0, 16)   # overlaps the GPU work
    w_gpu = weights.synthetic_experts(E, H, I, 0, DEV)
    ids, wts, off, pairs = native.moe_route_topk(torch.from_numpy(logits).to(DEV), k)
    assert np.array_equal(to_np(ids), rids)
    ws = _ffn_ws(T, H, I, E, k, native.W4A4)
    y, g_out = native.moe_grouped_nvfp4_ffn(x.to(DEV), w_gpu, ids, wts, off, pairs, k,
                                            act=native.W4A4, out_dtype=torch.float32,
                                            workspace=ws)
    torch.cuda.synchronize()
    hq_online = native.ffn_debug_h(ws, T, H, I, E, k, native.W4A4)[1].clone()
    ws2 = _ffn_ws(T, H, I, E, k, native.W4A4)
    y2, _ = native.moe_grouped_nvfp4_ffn(x.to(DEV), w_gpu, ids, wts, off, pairs, k,
                                         act=native.W4A4, act_globals=g_out.clone(),
                                         out_dtype=torch.float32, workspace=ws2)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "static g_h (fused epilogue) differs from the online step"
    hq_given = native.ffn_debug_h(ws2, T, H, I, E, k, native.W4A4, given=True)[1]
    kept = to_np(pairs) >= 0
    assert np.array_equal(to_np(hq_given)[kept], to_np(hq_online)[kept])
    w_ref = fut.result()
    pool.shutdown()
    _w4a4_device_h_check(x, rids, rw, w_ref, (ids, wts, off, pairs, w_gpu), y, g_out, T, H, I,
                         E, k, tokens=tokens, ws=ws)


@pytest.mark.parametrize("M", [512, 2048])
def test_dense_mlp_prefill_full_size_sampled(M):
    wl = synth.WORKLOADS[f"mlp_prefill_m{M}"]
    say("dense mlp prefill full size", M)
    x, rids, rw, y, _, w_ref, _ = _moe_run(wl.T, wl.H, wl.I, 1, 1)
    rows = [0, 1, M // 2 + 3, M - 1]   # first and last m-blocks, a middle one
    ref, _ = O.moe_ffn(x.float().numpy(), rids, rw, w_ref, tokens=rows)
    assert_close_f32(to_np(y)[rows], ref, "dense mlp prefill")


def test_dense_gemv_mlp_writes_y_with_dropped_rows():
    """One expert on the dense GEMV: the down projection's reduce writes y
    itself and the x pass zeroes the rows of tokens whose id is dropped (-1,
    or 1 with E = 1); kept rows match the oracle in fp32 and as its bf16
    rounding, dropped rows are 0 (y is filled with NaN first)."""
    import bench
    T, H, I = 8, 512, 768
    assert bench.gate_up_kernel(T, H, I, 1, 1, "w4a16") == "dense_gemv_kernel"
    say("dense gemv, dropped rows", T, H, I)
    x = synth.activations(T, H, 3)
    ids = np.zeros((T, 1), dtype=np.int32)
    ids[1, 0], ids[5, 0], ids[6, 0] = -1, -1, 1
    wts = np.ones((T, 1), dtype=np.float32)
    ids_t, wts_t = torch.from_numpy(ids).to(DEV), torch.from_numpy(wts).to(DEV)
    off, pairs = native.moe_permute_pairs(ids_t, 1)
    w_gpu = weights.synthetic_experts(1, H, I, 3, DEV)
    ys = {}
    for dt in (torch.float32, torch.bfloat16):
        y = torch.full((T, H), float("nan"), dtype=dt, device=DEV)
        native.moe_grouped_nvfp4_ffn(x.to(DEV), w_gpu, ids_t, wts_t, off, pairs, 1,
                                     out_dtype=dt, out=y)
        ys[dt] = to_np(y.float())
        assert np.all(ys[dt][[1, 5, 6]] == 0.0), dt
    ref, _ = O.moe_ffn(x.float().numpy(), ids, wts, oracle_experts(1, H, I, [0], 3))
    keep = [0, 2, 3, 4, 7]
    assert_close_f32(ys[torch.float32][keep], ref[keep], "dense gemv kept rows")
    assert_bf16_output(ys[torch.bfloat16][keep], ys[torch.float32][keep], ref[keep],
                       "dense gemv kept rows (bf16)")


@pytest.mark.parametrize("T,H,I", [(3, 256, 256), (16, 1024, 768), (17, 512, 2304),
                                   (32, 2048, 512), (5, 768, 1280)])
def test_dense_mlp_bf16_gemv_shapes(T, H, I):
    """A dense MLP of 3 to 32 rows on the bf16 GEMV (x and h as given, the
    weights dequantised to bf16): one and two 16-row subtiles (17 rows: a
    second subtile with one row), one-chunk K (256) and K splits over
    several owners per tile; fp32 output against the oracle's dense MLP and
    bf16 output as its rounding."""
    import bench
    assert bench.gate_up_kernel(T, H, I, 1, 1, "w4a16") == "dense_gemv_kernel"
    say("dense mlp bf16 gemv", T, H, I)
    x, rids, rw, y, _, w_ref, st = _moe_run(T, H, I, 1, 1, seed=T + H)
    ref = O.dense_mlp(x.float().numpy(), (w_ref.gate_codes[0], w_ref.gate_scales[0], w_ref.gate_global[0]),
                      (w_ref.up_codes[0], w_ref.up_scales[0], w_ref.up_global[0]),
                      (w_ref.down_codes[0], w_ref.down_scales[0], w_ref.down_global[0]))
    assert_close_f32(to_np(y), ref, "dense mlp bf16 gemv")
    ids, wts, off, pairs, w_gpu = st
    yb, _ = native.moe_grouped_nvfp4_ffn(x.to(DEV), w_gpu, ids, wts, off, pairs, 1,
                                         out_dtype=torch.bfloat16)
    assert_bf16_output(to_np(yb.float()), to_np(y), ref, "dense mlp bf16 gemv (bf16)")


@pytest.mark.parametrize("M", [1, 8, 32])
def test_dense_mlp_decode_full_size(M):
    """The dense NVFP4 MLP decode at full size, every row."""
    wl = synth.WORKLOADS[f"mlp_decode_m{M}"]
    say("dense mlp decode full size", M)
    x, rids, rw, y, _, w_ref, _ = _moe_run(wl.T, wl.H, wl.I, 1, 1)
    ref, _ = O.moe_ffn(x.float().numpy(), rids, rw, w_ref)
    assert_close_f32(to_np(y), ref, "dense mlp decode")


# ---------------------------------------------------------------------------
# empty batches: every batch call accepts T = 0 (routing sets its offsets to
# zero, the rest computes nothing) and the calls after it are unaffected
# ---------------------------------------------------------------------------

def test_empty_batch():
    E, H, I, k = 16, 256, 128, 4
    say("empty batch", E, H, I, k)
    i32 = dict(dtype=torch.int32, device=DEV)
    w = weights.synthetic_experts(E, H, I, 0, DEV)
    x0 = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    ids0, wts0 = torch.empty((0, k), **i32), torch.empty((0, k), dtype=torch.float32, device=DEV)
    pairs0 = torch.empty(0, **i32)
    off = torch.full((E + 1,), 7, **i32)
    native.moe_route_topk(torch.empty((0, E), dtype=torch.float32, device=DEV), k,
                          out=(ids0, wts0, off, pairs0))
    torch.cuda.synchronize()
    assert torch.equal(off, torch.zeros_like(off))
    rw = synth.router_matrix(E, H).to(DEV)
    off.fill_(7)
    native.moe_router_topk(x0, rw, k, out=(ids0, wts0, off, pairs0))
    torch.cuda.synchronize()
    assert torch.equal(off, torch.zeros_like(off))
    off.fill_(7)
    native.moe_permute_pairs(ids0, E, out=(off, pairs0))
    torch.cuda.synchronize()
    assert torch.equal(off, torch.zeros_like(off))
    for act in (native.W4A16, native.W4A4):
        y, _ = native.moe_grouped_nvfp4_ffn(x0, w, ids0, wts0, off, pairs0, k, act=act)
        assert y.shape == (0, H)
    # routing + FFN in one call (its decode shapes need H = 2048)
    x0d = torch.empty((0, 2048), dtype=torch.bfloat16, device=DEV)
    wd = weights.synthetic_experts(E, 2048, 256, 0, DEV, experts=[0])
    off.fill_(7)
    yd, _ = native.moe_route_ffn_decode(torch.empty((0, E), dtype=torch.float32, device=DEV), x0d,
                                        wd, k, route_out=(ids0, wts0, off, pairs0))
    torch.cuda.synchronize()
    assert yd.shape == (0, 2048) and torch.equal(off, torch.zeros_like(off))
    sh = [t.to(DEV) for t in synth.shared_expert_weights(H, I)]
    assert native.moe_shared_expert_ffn(x0, *sh).shape == (0, H)
    yl, _ = native.nvfp4_linear(x0, w.gate_codes[0], w.gate_scales[0], w.gate_global[:1])
    assert yl.shape == (0, I)
    # the slot plan of an empty step fetches nothing and moves nothing
    host = native.ExpertWeights(*[t.cpu().pin_memory() for t in (
        w.gate_codes, w.gate_scales, w.gate_global, w.up_codes, w.up_scales, w.up_global,
        w.down_codes, w.down_scales, w.down_global)])
    cache = native.ExpertCache(host, 8, DEV)
    first = torch.tensor([[1, 2, 3, 4]], **i32)
    cache.plan_and_fetch(first)
    torch.cuda.synchronize()
    state = (cache.slot_of.clone(), cache.expert_of.clone(), cache.hand.clone())
    cache.n_fetch.fill_(5)
    cache.plan_and_fetch(ids0)
    torch.cuda.synchronize()
    assert int(cache.n_fetch.item()) == 0
    assert all(torch.equal(a, b) for a, b in zip(state, (cache.slot_of, cache.expert_of,
                                                          cache.hand)))
    # a normal batch afterwards
    T = 9
    x = synth.activations(T, H, 3)
    logits = synth.router_logits(T, E, 3)
    rids, rwts = O.route_topk(logits, k)
    ids, wts, off, pairs = native.moe_route_topk(torch.from_numpy(logits).to(DEV), k)
    assert np.array_equal(to_np(ids), rids)
    y, _ = native.moe_grouped_nvfp4_ffn(x.to(DEV), w, ids, wts, off, pairs, k,
                                        out_dtype=torch.float32)
    ref, _ = O.moe_ffn(x.float().numpy(), rids, rwts, oracle_experts(E, H, I, np.unique(rids), 0))
    assert_close_f32(to_np(y), ref, "after an empty batch")
