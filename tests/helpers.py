"""Shared helpers for the parity tests: oracle-side weight preparation from
the same seeded fp32 weights the GPU side quantises, and the error metrics."""
from __future__ import annotations

import concurrent.futures

import numpy as np

from nvfp4_routed_expert_amd import synth
from oracle import nvfp4_oracle as O


class LazyOracleExperts(O.ExpertWeights):
    """Oracle ExpertWeights that quantises only the experts it is given."""

    def __init__(self, E, H, I, experts, seed=0, workers=8):
        experts = sorted(set(int(e) for e in experts))
        z = lambda *s: np.zeros(s, np.uint8)
        gc, gs, uc, us = z(E, I, H // 2), z(E, I, H // 16), z(E, I, H // 2), z(E, I, H // 16)
        dc, ds = z(E, H, I // 2), z(E, H, I // 16)
        gg, ug, dg = (np.ones(E, np.float32) for _ in range(3))

        def prep(e):
            g, u, d = synth.expert_weights_f32(e, H, I, seed)
            return e, O.quantize(g), O.quantize(u), O.quantize(d)

        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            for e, qg, qu, qd in ex.map(prep, experts):
                gc[e], gs[e], gg[e] = qg
                uc[e], us[e], ug[e] = qu
                dc[e], ds[e], dg[e] = qd
        super().__init__(gc, gs, gg, uc, us, ug, dc, ds, dg)
        self.filled = experts


def rel_frob(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def max_abs_over_rms(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(got - ref)) / max(rms, 1e-300))


# Output tolerance against the fp64 oracle (fp32 outputs): relative
# Frobenius error <= 1e-3 and max |error| <= 1e-2 * RMS of the reference.
REL_FROB_TOL = 1e-3
MAX_ABS_RMS_TOL = 1e-2


def assert_close_f32(got, ref, what=""):
    rf, ma = rel_frob(got, ref), max_abs_over_rms(got, ref)
    assert rf <= REL_FROB_TOL and ma <= MAX_ABS_RMS_TOL, \
        f"{what}: rel_frob={rf:.3e} max_abs/rms={ma:.3e}"
    return rf, ma


def bf16_ulp(v):
    """Spacing of bf16 at each |v| (fp64)."""
    v = np.abs(np.asarray(v, np.float64))
    _, e = np.frexp(np.where(v > 0, v, 1.0))
    return np.exp2(np.maximum(e, -125) - 8.0)


def assert_bf16_output(got_bf16, got_f32, ref64, what=""):
    """bf16 output: exactly the RNE rounding of the same kernel's fp32
    output; every element within max(one bf16 ulp, 1e-2 * RMS) of the
    rounded oracle value (a one-ulp flip where the fp32 sum and the fp64
    value straddle a rounding boundary is valid); and within the Frobenius
    bound of the rounded oracle."""
    g = np.asarray(got_bf16, np.float64)
    assert np.array_equal(g, O.bf16_rne(np.asarray(got_f32, np.float64))), \
        f"{what}: bf16 output is not the rounding of the fp32 output"
    r = O.bf16_rne(ref64)
    rms = float(np.sqrt(np.mean(np.asarray(ref64, np.float64) ** 2)))
    bound = np.maximum(bf16_ulp(r) * 1.0000001, MAX_ABS_RMS_TOL * rms)
    assert np.all(np.abs(g - r) <= bound), f"{what}: element beyond max(1 ulp, 1e-2 RMS)"
    assert rel_frob(g, r) <= REL_FROB_TOL, f"{what}: rel_frob {rel_frob(g, r):.3e}"


def spread_tokens(rids, n):
    """n tokens spread over the batch: one from each of n equal windows of
    token indices, each the token of its window that adds the fewest experts
    not yet chosen (so the oracle quantises fewer experts)."""
    rids = np.asarray(rids)
    chosen, have = [], set()
    for win in np.array_split(np.arange(rids.shape[0]), n):
        best = min(win, key=lambda t: (len(set(rids[t].tolist()) - have), t))
        chosen.append(int(best))
        have |= set(rids[best].tolist())
    return chosen


def rows_by_pair(rows_by_pos, sorted_pairs, P):
    """[P, I] rows indexed by pair from rows indexed by expert-sorted
    position (positions holding pair -1 are skipped; unfilled rows NaN)."""
    rows_by_pos = np.asarray(rows_by_pos, dtype=np.float64)
    sp = np.asarray(sorted_pairs)
    out = np.full((P, rows_by_pos.shape[1]), np.nan)
    kept = sp >= 0
    out[sp[kept]] = rows_by_pos[:len(sp)][kept]
    return out


def check_device_h(x32, rids, rw, w_ref, h_dev_pairs, hq_dev_pairs, g_x, g_h, tokens, act_quant,
                   y_dev_rows, what=""):
    """Several-results-correct check of a device's h, then everything after it.

    h_dev_pairs: the device's bf16 h [P, I] by pair (fp32 values); hq_dev_pairs:
    its W4A4 operand rows [P, I] (e2m1*e4m3, without g_h) or None.  For the
    sampled tokens' kept pairs:
      1. every device h value is a valid rounding of the fp64 h (the exact
         bf16 rounding, or either neighbour where the fp32 error bound reaches
         the rounding boundary: O.check_h_choices);
      2. W4A4: the operand rows are exactly the oracle's quantisation of the
         device's h with the device's g_h;
      3. the device's output rows meet the fp32 tolerance against the oracle
         computed downstream from the device's h.
    Returns (flips, flagged, values checked)."""
    ids = np.asarray(rids)
    n_exp = w_ref.gate_codes.shape[0]
    k = ids.shape[1]
    tokens = np.asarray(tokens)
    pair_idx = tokens[:, None] * k + np.arange(k)[None, :]           # [n, k]
    h_given = np.asarray(h_dev_pairs, dtype=np.float64)[pair_idx]     # [n, k, I]
    ag = (g_x, g_h) if act_quant else None
    ref, info = O.moe_ffn(x32, ids, rw, w_ref, act_quant=act_quant, act_globals=ag,
                          tokens=tokens, h_given=h_given, with_bound=True)
    kept = info["kept"]
    ok, flagged, flips = O.check_h_choices(info["h64"][kept], info["h_bound"][kept],
                                           h_given[kept])
    assert ok.all(), (f"{what}: {int((~ok).sum())} device h values are not a valid rounding "
                      f"of the fp64 h")
    if act_quant and hq_dev_pairs is not None:
        hq = np.asarray(hq_dev_pairs, dtype=np.float64)[pair_idx][kept]
        hc, hs, _ = O.quantize(h_given[kept].astype(np.float32), g_h)
        assert np.array_equal(hq, O.block_values(hc, hs)), f"{what}: h operand codes differ"
    assert_close_f32(y_dev_rows, ref, what)
    return int(flips.sum()), int(flagged.sum()), int(flips.size)
