"""Pins of the oracle's linear map, routing, permutation and expert FFN."""
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

from oracle import nvfp4_oracle as O


def _frac(v):
    return Fraction(float(v))


def _rand_nvfp4(rng, n, k):
    codes = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = rng.integers(0x20, 0x48, size=(n, k // 16), dtype=np.uint8)
    return codes, scales


def test_linear_exact_rationals():
    rng = np.random.default_rng(0)
    m, n, k = 3, 5, 32
    codes, scales = _rand_nvfp4(rng, n, k)
    g = np.float32(0.0078125 * 3)                     # dyadic * 3
    x = (rng.integers(-64, 64, size=(m, k)) / 16.0).astype(np.float32)
    y, _ = O.linear(x, codes, scales, g)
    el = O.unpack_nibbles(codes)
    table = {c: _frac(v) for c, v in enumerate(O.decode_e2m1(np.arange(16)))}
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for kk in range(k):
                s = _frac(O.decode_e4m3(scales[j, kk // 16]))
                acc += _frac(x[i, kk]) * table[int(el[j, kk])] * s
            exact = acc * _frac(g)
            assert abs(_frac(y[i, j]) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)


def test_linear_all_ones_gives_row_sums():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 64)).astype(np.float32)
    codes = np.full((3, 32), 0x22, np.uint8)          # every element code 2 = 1.0
    scales = np.full((3, 4), 0x38, np.uint8)          # every scale 1.0
    y, _ = O.linear(x, codes, scales, np.float32(1.0))
    assert np.allclose(y, x.astype(np.float64).sum(1)[:, None], rtol=1e-14, atol=1e-14)


def test_linear_one_hot_picks_columns():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 32)).astype(np.float32)
    el = np.zeros((32, 32), np.uint8)
    for j in range(32):
        el[j, (5 * j) % 32] = 2                       # 1.0 at column (5j mod 32)
    codes = O.pack_nibbles(el)
    scales = np.full((32, 2), 0x38, np.uint8)
    y, _ = O.linear(x, codes, scales, np.float32(0.5))
    assert np.array_equal(y, 0.5 * x.astype(np.float64)[:, (5 * np.arange(32)) % 32])


def test_linear_w4a4_is_linear_on_dequantised_activations():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, 64)).astype(np.float32)
    codes, scales = _rand_nvfp4(rng, 8, 64)
    y, gx = O.linear(x, codes, scales, np.float32(0.01), act_quant=True)
    xc, xs, gx2 = O.quantize(x)
    assert gx == gx2
    y2, _ = O.linear(O.dequantize(xc, xs, gx), codes, scales, np.float32(0.01))
    assert np.allclose(y, y2, rtol=1e-12, atol=0)


def _check_topk_characterisation(logits, ids):
    t, e = logits.shape
    for i in range(t):
        chosen = list(ids[i])
        assert len(set(chosen)) == len(chosen)
        key = lambda j: (-float(logits[i, j]), j)
        # listed in order, and every chosen expert beats every other one
        assert [key(j) for j in chosen] == sorted(key(j) for j in chosen)
        rest = [j for j in range(e) if j not in chosen]
        if rest:
            assert max(key(j) for j in chosen) < min(key(j) for j in rest)


@pytest.mark.parametrize("seed", range(5))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    t, e, k = 8, 16, 4
    logits = rng.integers(-3, 3, size=(t, e)).astype(np.float32)  # many ties
    ids, w = O.route_topk(logits, k)
    _check_topk_characterisation(logits, ids)
    # brute force over all k-subsets: the chosen set maximises the logit sum,
    # and among maximisers is the lexicographically smallest sorted index set
    from itertools import combinations
    for i in range(t):
        best = max(combinations(range(e), k),
                   key=lambda c: (sum(float(logits[i, j]) for j in c), [-j for j in c]))
        assert sorted(ids[i]) == sorted(best)
    assert np.allclose(w.sum(1), 1.0, atol=1e-15)


def test_topk_weights_are_renormalised_softmax():
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((5, 12)).astype(np.float32)
    ids, w = O.route_topk(logits, 3)
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    assert np.allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-13)
    ids2, w2 = O.route_topk(logits, 3, renormalize=False)
    assert np.array_equal(ids, ids2) and np.allclose(w2, sel, rtol=1e-13)
    # k = E with renormalisation is the softmax itself
    ids3, w3 = O.route_topk(logits, 12)
    full = np.take_along_axis(p, ids3.astype(np.int64), axis=1)
    assert np.allclose(w3, full, rtol=1e-13)


def test_permute_invariants():
    rng = np.random.default_rng(4)
    t, e, k = 37, 10, 3
    ids, _ = O.route_topk(rng.standard_normal((t, e)).astype(np.float32), k)
    offsets, pairs = O.permute(ids, e)
    assert offsets[0] == 0 and offsets[-1] == t * k
    assert np.all(np.diff(offsets) >= 0)
    assert np.array_equal(np.sort(pairs), np.arange(t * k))
    flat = ids.reshape(-1)
    for ex in range(e):
        seg = pairs[offsets[ex]:offsets[ex + 1]]
        assert np.all(flat[seg] == ex)
        assert np.all(np.diff(seg // k) > 0)          # ascending tokens
        assert len(seg) == np.count_nonzero(flat == ex)


def _rand_experts(rng, e, h, i):
    def q(n, kk):
        return O.quantize((rng.standard_normal((n, kk)) * 0.05).astype(np.float32))
    mats = [[q(i, h) for _ in range(e)], [q(i, h) for _ in range(e)],
            [q(h, i) for _ in range(e)]]
    stack = lambda lst, j: np.stack([m[j] for m in lst])
    return O.ExpertWeights(stack(mats[0], 0), stack(mats[0], 1), stack(mats[0], 2),
                           stack(mats[1], 0), stack(mats[1], 1), stack(mats[1], 2),
                           stack(mats[2], 0), stack(mats[2], 1), stack(mats[2], 2))


def test_moe_single_expert_is_dense_mlp_from_linear():
    rng = np.random.default_rng(5)
    t, h, i = 6, 64, 32
    w = _rand_experts(rng, 1, h, i)
    x = rng.standard_normal((t, h)).astype(np.float32)
    y, _ = O.moe_ffn(x, np.zeros((t, 1), np.int32), np.ones((t, 1)), w)
    gate, _ = O.linear(x, w.gate_codes[0], w.gate_scales[0], w.gate_global[0])
    up, _ = O.linear(x, w.up_codes[0], w.up_scales[0], w.up_global[0])
    hh = O.bf16_rne(gate / (1 + np.exp(-gate)) * up)
    y2, _ = O.linear(hh, w.down_codes[0], w.down_scales[0], w.down_global[0])
    assert np.allclose(y, y2, rtol=1e-12, atol=1e-15)


def test_moe_equal_logits_all_experts_is_mean():
    rng = np.random.default_rng(6)
    t, h, i, e = 4, 32, 32, 4
    w = _rand_experts(rng, e, h, i)
    x = rng.standard_normal((t, h)).astype(np.float32)
    ids, wts = O.route_topk(np.zeros((t, e), np.float32), e)
    assert np.array_equal(ids, np.tile(np.arange(e), (t, 1)))
    assert np.allclose(wts, 1.0 / e)
    y, _ = O.moe_ffn(x, ids, wts, w)
    per = []
    for ex in range(e):
        ye, _ = O.moe_ffn(x, np.full((t, 1), ex, np.int32), np.ones((t, 1)), w)
        per.append(ye)
    assert np.allclose(y, np.mean(per, axis=0), rtol=1e-12, atol=1e-15)


def test_moe_token_subset_matches_full():
    rng = np.random.default_rng(7)
    t, h, i, e, k = 12, 32, 32, 6, 2
    w = _rand_experts(rng, e, h, i)
    x = rng.standard_normal((t, h)).astype(np.float32)
    ids, wts = O.route_topk(rng.standard_normal((t, e)).astype(np.float32), k)
    y, _ = O.moe_ffn(x, ids, wts, w)
    ys, _ = O.moe_ffn(x, ids, wts, w, tokens=[3, 0, 11])
    assert np.array_equal(ys, y[[3, 0, 11]])


def test_moe_w4a4_single_expert_composes_quantised_linears():
    rng = np.random.default_rng(8)
    t, h, i = 5, 64, 32
    w = _rand_experts(rng, 1, h, i)
    x = rng.standard_normal((t, h)).astype(np.float32)
    y, info = O.moe_ffn(x, np.zeros((t, 1), np.int32), np.ones((t, 1)), w,
                        act_quant=True)
    gate, gx = O.linear(x, w.gate_codes[0], w.gate_scales[0], w.gate_global[0], act_quant=True)
    up, _ = O.linear(x, w.up_codes[0], w.up_scales[0], w.up_global[0], act_quant=True)
    hh = O.bf16_rne(gate / (1 + np.exp(-gate)) * up)
    y2, gh = O.linear(hh.astype(np.float32), w.down_codes[0], w.down_scales[0],
                      w.down_global[0], act_quant=True)
    assert info["g_x"] == gx and info["g_h"] == gh
    assert np.allclose(y, y2, rtol=1e-12, atol=1e-15)
    # given globals reproduce the computed ones
    y3, _ = O.moe_ffn(x, np.zeros((t, 1), np.int32), np.ones((t, 1)), w,
                      act_quant=True, act_globals=(gx, gh), tokens=[1, 4])
    assert np.array_equal(y3, y[[1, 4]])


def _bf16_boundary_distance(v):
    """Relative distance of each fp64 v from the nearest bf16 rounding
    boundary (midpoint between neighbouring bf16 values)."""
    v = np.abs(np.asarray(v, np.float64))
    _, e = np.frexp(np.where(v > 0, v, 1.0))
    q = np.exp2(np.maximum(e, -125) - 8.0)          # bf16 spacing at v
    frac = v / q - np.floor(v / q)                  # position between neighbours
    return np.abs(frac - 0.5) * q / np.where(v > 0, v, 1.0)


@pytest.mark.parametrize("act_quant", [False, True])
def test_moe_fp32_h_differs_from_fp64_h_only_next_to_bf16_ties(act_quant):
    """The fp32 h agrees with the fp64 h, which the tests above pin, except
    where the fp64 value before its bf16 rounding lies within fp32 rounding
    error of a rounding boundary; there the two are neighbouring bf16
    values.  A swapped gate/up, a dropped global or a wrong operand would
    change most elements."""
    rng = np.random.default_rng(21)
    t, h, i = 2000, 64, 256          # 512000 h values: a few sit next to a tie
    w = _rand_experts(rng, 1, h, i)
    x = rng.standard_normal((t, h)).astype(np.float32)
    ids, wts = np.zeros((t, 1), np.int32), np.ones((t, 1))
    _, i64 = O.moe_ffn(x, ids, wts, w, act_quant=act_quant)
    _, i32 = O.moe_ffn(x, ids, wts, w, act_quant=act_quant, h_fp32=True)
    h64, h32 = i64["h_bf16"][:, 0], i32["h_bf16"][:, 0]
    # the fp64 value before rounding, from the pinned linear maps
    gate, _ = O.linear(x, w.gate_codes[0], w.gate_scales[0], w.gate_global[0], act_quant=act_quant)
    up, _ = O.linear(x, w.up_codes[0], w.up_scales[0], w.up_global[0], act_quant=act_quant)
    pre = gate / (1 + np.exp(-gate)) * up
    assert np.array_equal(O.bf16_rne(pre), h64)
    diff = h32 != h64
    assert 0 < diff.sum() <= 20
    assert np.all(_bf16_boundary_distance(pre[diff]) < 2.0 ** -18)
    ulp = np.exp2(np.frexp(np.maximum(np.abs(h32[diff]), np.abs(h64[diff])))[1] - 8.0)
    assert np.all(np.abs(h32[diff] - h64[diff]) <= ulp)


def test_moe_fp32_h_closed_forms():
    """Single expert, one nonzero column: gate = 40 makes exp(-gate) vanish
    next to 1 in fp32, so h = gate * up exactly; gate = -200 overflows exp
    and gives h = 0; a zero gate gives h = 0."""
    h, i = 16, 16
    codes = np.zeros((i, h), np.uint8)
    codes[:, 0] = 2                                  # e2m1 code 2 = 1.0
    scales = np.full((i, 1), 0x38, np.uint8)         # e4m3 0x38 = 1.0
    pk = O.pack_nibbles(codes)

    def experts(g_gate, g_up):
        return O.ExpertWeights(pk[None], scales[None], np.array([g_gate], np.float32),
                               pk[None], scales[None], np.array([g_up], np.float32),
                               pk[None].reshape(1, h, i // 2), scales[None].reshape(1, h, 1),
                               np.array([1.0], np.float32))

    x = np.zeros((3, h), np.float32)
    x[:, 0] = [2.0, -10.0, 0.0]
    ids, wts = np.zeros((3, 1), np.int32), np.ones((3, 1))
    _, info = O.moe_ffn(x, ids, wts, experts(20.0, 1.5), h_fp32=True)
    hb = info["h_bf16"][:, 0]
    assert np.all(hb[0] == 2.0 * 20.0 * 2.0 * 1.5)   # gate 40, up 6 -> 240
    assert np.all(hb[1] == 0.0)                        # gate -200, up -30
    assert np.all(hb[2] == 0.0)


def test_router_logits_exact_on_small_rationals():
    """Brute force with exact rationals: every product and the bias."""
    from fractions import Fraction
    x = np.array([[1.0, -2.0, 0.5, 0.25], [3.0, 0.0, -1.0, 2.0]], np.float32)
    r = np.array([[0.5, 0.5, 1.0, -4.0], [2.0, -1.0, 0.0, 1.0], [0.0, 0.0, 0.0, 0.0]],
                 np.float32)
    bias = np.array([0.0, -1.5, 0.125], np.float32)
    lg = O.router_logits(x, r, bias)
    for t in range(2):
        for e in range(3):
            want = sum(Fraction(float(x[t, h])) * Fraction(float(r[e, h])) for h in range(4))
            assert Fraction(lg[t, e]) == want + Fraction(float(bias[e]))
    assert lg[1, 0] == 1.5 - 1.0 - 8.0
    assert np.array_equal(O.router_logits(x, r), lg - bias[None, :])


def test_router_logits_one_hot_rows_pick_router_columns():
    rng = np.random.default_rng(9)
    r = rng.standard_normal((5, 8)).astype(np.float32)
    x = np.eye(8, dtype=np.float32)[[3, 0, 7]]
    assert np.array_equal(O.router_logits(x, r), r.T[[3, 0, 7]].astype(np.float64))


def test_shared_expert_is_the_one_expert_ffn_on_exact_weights():
    """With bf16 weights that are exact NVFP4 values (the dequantised
    matrices of a one-expert FFN), the shared expert equals the routed FFN
    with that single expert and weight 1, which the tests above pin."""
    rng = np.random.default_rng(12)
    t, h, i = 7, 64, 96
    w = _rand_experts(rng, 1, h, i)
    x = O.bf16_rne(rng.standard_normal((t, h))).astype(np.float32)
    wg = O.dequantize(w.gate_codes[0], w.gate_scales[0], w.gate_global[0])
    wu = O.dequantize(w.up_codes[0], w.up_scales[0], w.up_global[0])
    wd = O.dequantize(w.down_codes[0], w.down_scales[0], w.down_global[0])
    y_moe, _ = O.moe_ffn(x, np.zeros((t, 1), np.int32), np.ones((t, 1)), w)
    y = O.shared_expert(x, wg, wu, wd)
    assert np.allclose(y, y_moe, rtol=1e-12, atol=1e-15)
    # accumulate adds the given output
    y_in = rng.standard_normal((t, h))
    assert np.array_equal(O.shared_expert(x, wg, wu, wd, y_in), y_in + y)


def test_shared_expert_closed_form():
    """Gate row = 10 e_0 (silu is then 10 up to 5e-4), up row = e_1, down = I:
    h = bf16(silu(10 x_0) x_1), y = h."""
    x = np.array([[1.0, 3.0, 0.0, 0.0], [-1.0, 2.0, 0.0, 0.0]], np.float32)
    wg = np.zeros((4, 4)); wg[:, 0] = 10.0
    wu = np.zeros((4, 4)); wu[:, 1] = 1.0
    wd = np.eye(4)
    y = O.shared_expert(x, wg, wu, wd)
    s0 = 10.0 / (1 + np.exp(-10.0))
    s1 = -10.0 / (1 + np.exp(10.0))
    assert np.all(y[0] == O.bf16_rne(s0 * 3.0))
    assert np.all(y[1] == O.bf16_rne(s1 * 2.0))


# ---------------------------------------------------------------------------
# dropped pairs (ids outside 0..E-1), given h, and the valid roundings of h
# ---------------------------------------------------------------------------

def test_permute_drops_ids_outside_the_experts():
    rng = np.random.default_rng(31)
    t, e, k = 23, 7, 3
    ids, _ = O.route_topk(rng.standard_normal((t, e)).astype(np.float32), k)
    full_off, full_pairs = O.permute(ids, e)
    drop = rng.random((t, k)) < 0.3
    ids_d = np.where(drop, np.where(rng.random((t, k)) < 0.5, -1, e), ids)
    off, pairs = O.permute(ids_d, e)
    kept = int((~drop).sum())
    assert off[-1] == kept and np.all(pairs[kept:] == -1)
    # the kept pairs keep the relative order of the full permutation
    keep_flat = ~drop.reshape(-1)
    assert np.array_equal(pairs[:kept], full_pairs[keep_flat[full_pairs]])
    assert np.array_equal(np.diff(off), np.bincount(ids_d[~drop], minlength=e))


def test_moe_dropped_pairs_contribute_nothing():
    """W4A16: a dropped pair gives the same output as a kept pair with routing
    weight 0 (adding an exact zero changes no fp64 sum); a token whose pairs
    are all dropped gets 0."""
    rng = np.random.default_rng(32)
    t, h, i, e, k = 9, 32, 32, 5, 3
    w = _rand_experts(rng, e, h, i)
    x = rng.standard_normal((t, h)).astype(np.float32)
    ids, wts = O.route_topk(rng.standard_normal((t, e)).astype(np.float32), k)
    drop = rng.random((t, k)) < 0.4
    drop[4] = True
    y_d, info = O.moe_ffn(x, np.where(drop, -1, ids), wts, w)
    y_0, _ = O.moe_ffn(x, ids, np.where(drop, 0.0, wts), w)
    assert np.array_equal(y_d, y_0)
    assert np.all(y_d[4] == 0) and np.array_equal(info["kept"], ~drop)


def test_moe_w4a4_dropped_pairs_take_no_part_in_the_h_scale():
    """W4A4 online: dropping every pair of the second half of the tokens
    gives, for the first half, exactly the call on those tokens alone with
    the full x's activation scale (the h scale then spans the same pairs),
    and zeros for the second half."""
    rng = np.random.default_rng(33)
    t, h, i, e, k = 10, 64, 32, 4, 2
    w = _rand_experts(rng, e, h, i)
    x = rng.standard_normal((t, h)).astype(np.float32)
    ids, wts = O.route_topk(rng.standard_normal((t, e)).astype(np.float32), k)
    ids_d = ids.copy()
    ids_d[t // 2:] = -1
    y_d, info_d = O.moe_ffn(x, ids_d, wts, w, act_quant=True)
    g_x = O.tensor_global(x)
    y_h, info_h = O.moe_ffn(x[:t // 2], ids[:t // 2], wts[:t // 2], w, act_quant=True,
                            act_globals=(g_x, None))
    assert info_d["g_x"] == g_x and info_d["g_h"] == info_h["g_h"]
    assert np.array_equal(y_d[:t // 2], y_h) and np.all(y_d[t // 2:] == 0)


@pytest.mark.parametrize("act_quant", [False, True])
def test_moe_given_h_reproduces_the_computed_one(act_quant):
    rng = np.random.default_rng(34)
    t, h, i, e, k = 8, 64, 48, 5, 2
    w = _rand_experts(rng, e, h, i)
    x = rng.standard_normal((t, h)).astype(np.float32)
    ids, wts = O.route_topk(rng.standard_normal((t, e)).astype(np.float32), k)
    y, info = O.moe_ffn(x, ids, wts, w, act_quant=act_quant)
    y2, info2 = O.moe_ffn(x, ids, wts, w, act_quant=act_quant, h_given=info["h_bf16"])
    assert np.array_equal(y, y2) and np.array_equal(info["h"], info2["h"])
    # a different h changes the result: the given values are what is used
    other = info["h_bf16"].copy()
    other[0, 0, 0] += 1.0
    y3, _ = O.moe_ffn(x, ids, wts, w, act_quant=act_quant, h_given=other)
    assert not np.array_equal(y3[0], y[0])
    if not act_quant:   # (in W4A4 the larger h may also move the h scale)
        assert np.array_equal(y3[1:], y[1:])


def test_bf16_bracket():
    rng = np.random.default_rng(35)
    v = rng.standard_normal(20000) * np.exp2(rng.integers(-40, 40, 20000))
    v[:4] = [1.0, -1.5, 2.0 ** -130, 0.0]
    lo, hi = O.bf16_bracket(v)
    assert np.all(lo <= v) and np.all(v <= hi)
    assert np.array_equal(O.bf16_rne(lo), lo) and np.array_equal(O.bf16_rne(hi), hi)
    r = O.bf16_rne(v)
    assert np.all((r == lo) | (r == hi))
    exact = O.bf16_rne(v) == v
    assert np.array_equal(lo == hi, exact)
    # neighbours: nothing representable strictly between lo and hi
    mid = 0.5 * (lo + hi)
    assert np.all((O.bf16_rne(mid) == lo) | (O.bf16_rne(mid) == hi))


def test_check_h_choices_cases():
    one = 1.0
    mid = 1.0 + 2.0 ** -8                    # half-way between 1 and 1 + 2^-7
    up = 1.0 + 2.0 ** -7
    # exactly on the boundary: both neighbours valid; the rounding picks 1 (even)
    ok, fl, fp = O.check_h_choices([mid, mid], [0.0, 0.0], [one, up])
    assert ok.all() and fl.all() and fp.tolist() == [False, True]
    # off the boundary by more than the bound: only the rounding is valid
    v = mid + 2.0 ** -20
    ok, fl, _ = O.check_h_choices([v, v], [2.0 ** -22] * 2, [up, one])
    assert ok.tolist() == [True, False] and not fl.any()
    # within the bound: either neighbour
    ok, fl, _ = O.check_h_choices([v, v], [2.0 ** -19] * 2, [up, one])
    assert ok.all() and fl.all()
    # two ulps away is never valid; an exact bf16 value has one valid result
    ok, _, _ = O.check_h_choices([v, 1.5, 1.5], [1.0, 1.0, 1.0], [1.0 + 2.0 ** -6, 1.5, up])
    assert ok.tolist() == [False, True, False]
    # negative values mirror
    ok, fl, _ = O.check_h_choices([-mid], [0.0], [-up])
    assert ok.all() and fl.all()


def _fp32_h(xv, g_x, w, e, order, rng):
    """h of expert e evaluated in fp32 with a given summation order of the
    K products (each product is exact in fp32), then the fp32 globals,
    SiLU and product; bf16 rounding left out."""
    f32 = np.float32
    dg = O.block_values(w.gate_codes[e], w.gate_scales[e]).astype(f32)
    du = O.block_values(w.up_codes[e], w.up_scales[e]).astype(f32)
    xv = np.asarray(xv, f32)
    k = dg.shape[1]
    perm = np.arange(k)
    if order == "reversed":
        perm = perm[::-1]
    elif order == "random":
        perm = rng.permutation(k)

    def acc(d):
        if order == "blocked32":   # exact 32-term blocks, then fp32 accumulation
            s = np.zeros((xv.shape[0], d.shape[0]), f32)
            for b in range(0, k, 32):
                blk = (xv[:, b:b + 32].astype(np.float64) @ d[:, b:b + 32].T.astype(np.float64))
                s = (s + blk.astype(f32)).astype(f32)
            return s
        s = np.zeros((xv.shape[0], d.shape[0]), f32)
        for j in perm:
            s = (s + xv[:, j:j + 1] * d[None, :, j]).astype(f32)
        return s
    gx = f32(1.0) if g_x is None else f32(g_x)
    g = acc(dg) * (f32(w.gate_global[e]) * gx)
    u = acc(du) * (f32(w.up_global[e]) * gx)
    with np.errstate(over="ignore"):
        return ((g / (f32(1.0) + np.exp(-g))) * u).astype(np.float64)


@pytest.mark.parametrize("act_quant", [False, True])
def test_h_bound_covers_fp32_evaluations(act_quant):
    """The bound of expert_h_bound holds for fp32 evaluations of h in several
    summation orders (sequential, reversed, random, exact 32-term blocks),
    computed independently here; it stays far below the bf16 spacing for
    most values (so the rounding is decided almost everywhere)."""
    rng = np.random.default_rng(36)
    t, h, i = 48, 512, 64
    w = _rand_experts(rng, 1, h, i)
    x = O.bf16_rne(rng.standard_normal((t, h))).astype(np.float32)
    if act_quant:
        xc, xs, g_x = O.quantize(x)
        xv = O.block_values(xc, xs)
    else:
        xv, g_x = x.astype(np.float64), None
    h64, dh = O.expert_h_bound(xv, g_x, w, 0)
    # the fp64 h is the one moe_ffn rounds
    _, info = O.moe_ffn(x, np.zeros((t, 1), np.int32), np.ones((t, 1)), w, act_quant=act_quant,
                        with_bound=True)
    assert np.allclose(info["h64"][:, 0], h64, rtol=1e-12, atol=0)
    assert np.array_equal(O.bf16_rne(h64), info["h_bf16"][:, 0])
    worst = 0.0
    for order in ("sequential", "reversed", "random", "blocked32"):
        h32 = _fp32_h(xv, g_x, w, 0, order, rng)
        err = np.abs(h32 - h64)
        assert np.all(err <= dh), order
        worst = max(worst, float(np.max(err / np.where(dh > 0, dh, 1))))
    assert worst > 1e-3                     # the bound is not vacuous
    rel = dh / np.maximum(np.abs(h64), 1e-30)
    assert np.median(rel) < 2.0 ** -12      # far below bf16's half spacing (2^-9)
