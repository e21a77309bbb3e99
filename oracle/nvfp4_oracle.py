"""CPU oracle for the NVFP4 routed-expert FFN.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant generator with the HIP library, and it never consumes a value the
HIP library produced.

What it computes, in plain numpy (fp64 unless a step is defined in fp32):

* NVFP4 tensors.  A matrix W[N, K] is stored as 4-bit E2M1 codes, two per
  byte (Qwen3.8-Flash-Next-NVFP4-SSD-Stream model card, "Why Hugging Face
  shows 68B parameters and 8-bit precision": each packed byte holds two
  NVFP4 values), one FP8 E4M3 scale per 16 consecutive elements along K and
  one fp32 scale per tensor.  The element and scale encodings are the OCP
  Microscaling Formats (MX) v1.0 FP4 E2M1 and FP8 E4M3 element types; the
  pages name NVFP4 but do not define its bits.
* Weight-only (W4A16) and weight+activation (W4A4) linear maps; the routed
  experts of the Flash-Next NVFP4 checkpoint are W4A4 (same model card,
  "What this model is"), the DFlash2 drafter is weight-only
  (Qwen3.8-27B-nvfp4full-dflash2-NInfer model card, "Limits").
* The BF16 router's logits (a plain product), top-k routing over the
  experts, the expert-sorted pair permutation, the gated (SiLU) expert FFN
  with a routing-weighted combine and the BF16 shared expert (Eider page,
  "Qwen3.8 Flash Next": all 512 MoE experts; "Performance": prefill batches
  up to 512 prompt tokens so routed expert weights are reused).
* The slot plan of expert paging (``expert_slot_plan``): which experts a
  bounded device pool keeps, fetches and evicts in a step (Eider page, "Why
  Eider exists"); the FFN on the pool is the FFN above.

Readings where the pages are silent (each is a plain reading that the rest
of the pages supports): element 2i sits in the low nibble; scales are row-major
[N, K/16]; the fp32 tensor scale is the *decode* multiplier
g = amax / (6 * 448); block scales round to nearest-even E4M3 and saturate at
448; elements round to nearest-even E2M1 and saturate at +-6; the sign of a
zero code is kept; quantisation uses the fp32 operation order written in
``quantize``; ties in top-k go to the lower expert index; h is rounded to
bf16 before the down projection.  The pages fix no precision for forming h;
besides the fp64 h, ``expert_h_fp32`` forms it with fp32 operations (the
FFN's fp32 accumulation) for comparisons where h's bf16 rounding and NVFP4
codes must be decided in the same precision on both sides.  Where a device
computes h in fp32, ``expert_h_bound`` bounds its distance from the fp64 h
and ``check_h_choices`` tells which bf16 values of h are then valid: the
exact rounding, or either neighbour where the bound reaches the rounding
boundary (several results are correct there); ``moe_ffn(h_given=...)``
computes everything after h from such valid choices.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Element encodings (OCP MX v1.0 element types)
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0      # largest finite OCP E4M3 value, code 0x7E
E2M1_MAX = 6.0        # largest E2M1 magnitude, code 0x7
QUANT_RANGE = E2M1_MAX * E4M3_MAX   # 2688: amax maps onto the largest block scale


def decode_e2m1(codes):
    """Value of 4-bit E2M1 codes (OCP MX v1.0 FP4 E2M1).

    Bit 3 is the sign, bits 2..1 the exponent (bias 1), bit 0 the mantissa.
    Exponent field 0 is subnormal: m * 0.5.  Otherwise 2**(e-1) * (1 + m/2).
    """
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c > 15)):
        raise ValueError("E2M1 codes are 4-bit")
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, m * 0.5, np.exp2(e - 1.0) * (1.0 + m / 2.0))
    return np.where((c & 8) != 0, -mag, mag)


def decode_e4m3(codes):
    """Value of FP8 E4M3 bytes (OCP MX v1.0 FP8 E4M3, the 'FN' variant).

    Bit 7 is the sign, bits 6..3 the exponent (bias 7), bits 2..0 the
    mantissa.  Exponent field 0 is subnormal: m * 2**-9.  S.1111.111 is NaN;
    there is no infinity, so 448 is the largest finite value.
    """
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c > 255)):
        raise ValueError("E4M3 codes are bytes")
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, np.exp2(e - 7.0) * (1.0 + m / 8.0))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


# Every finite non-negative value of each type, ascending with its code.
_E2M1_POS_CODES = np.arange(8)
_E2M1_POS_VALUES = decode_e2m1(_E2M1_POS_CODES)
_E4M3_POS_CODES = np.arange(0x7F)          # 0x00 .. 0x7E (0x7F is NaN)
_E4M3_POS_VALUES = decode_e4m3(_E4M3_POS_CODES)


def _nearest_even(v, grid_values, grid_codes):
    """Index into an ascending grid of the value nearest to each v >= 0.

    Values above the grid saturate to its last entry.  When v lies exactly
    half-way between two neighbours, the neighbour whose code has a zero
    mantissa LSB (an even code) is taken: round-half-to-even.  All
    arithmetic is fp64 on fp32 inputs and dyadic grid points, so the
    distance comparison is exact.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or not np.all(np.isfinite(v)):
        raise ValueError("magnitudes must be finite and non-negative")
    hi = np.searchsorted(grid_values, v, side="left")     # first grid >= v
    hi = np.minimum(hi, len(grid_values) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = v - grid_values[lo]
    d_hi = grid_values[hi] - v
    pick_hi = np.where(d_hi < d_lo, True,
                       np.where(d_hi > d_lo, False, (grid_codes[hi] & 1) == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(v >= grid_values[-1], len(grid_values) - 1, idx)
    return idx


def e4m3_rne_saturate(v):
    """Nearest E4M3 code (ties to even mantissa) of v >= 0; v > 448 -> 0x7E."""
    idx = _nearest_even(v, _E4M3_POS_VALUES, _E4M3_POS_CODES)
    return _E4M3_POS_CODES[idx].astype(np.uint8)


def e2m1_rne_saturate(v):
    """Nearest E2M1 code of a signed value, ties to even mantissa, |v| > 6 -> 6.

    The sign bit is copied from v, so a negative value that rounds to zero
    gives code 0x8.
    """
    v = np.asarray(v, dtype=np.float64)
    idx = _nearest_even(np.abs(v), _E2M1_POS_VALUES, _E2M1_POS_CODES)
    code = _E2M1_POS_CODES[idx]
    code = np.where(np.signbit(v), code | 8, code)
    return code.astype(np.uint8)


# ---------------------------------------------------------------------------
# Packing (two E2M1 codes per byte, element 2i in the low nibble)
# ---------------------------------------------------------------------------

def pack_nibbles(codes):
    """[..., K] 4-bit codes -> [..., K/2] bytes; element 2i -> low nibble."""
    c = np.asarray(codes).astype(np.uint8)
    if c.shape[-1] % 2:
        raise ValueError("K must be even")
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """[..., K/2] bytes -> [..., K] 4-bit codes (low nibble first)."""
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


# ---------------------------------------------------------------------------
# Dequantisation: value = e2m1(code) * e4m3(block scale) * g
# ---------------------------------------------------------------------------

def block_values(codes_packed, scales):
    """fp64 e2m1(code) * e4m3(scale of its 16-block), without the tensor scale.

    codes_packed [N, K/2] uint8, scales [N, K/16] uint8 -> [N, K] float64.
    The product has at most 6 significant bits, so it is exact here.
    """
    e = decode_e2m1(unpack_nibbles(codes_packed))
    s = decode_e4m3(scales)
    n, k = e.shape
    if s.shape != (n, k // 16):
        raise ValueError(f"scales shape {s.shape} != {(n, k // 16)}")
    return e * np.repeat(s, 16, axis=1)


def dequantize(codes_packed, scales, g):
    """Dense fp64 matrix of an NVFP4 tensor: e2m1 * e4m3 * g."""
    return block_values(codes_packed, scales) * np.float64(np.float32(g))


def dequantize_f32(codes_packed, scales, g):
    """The dequantised matrix rounded once to fp32 (the debug output form)."""
    return dequantize(codes_packed, scales, g).astype(np.float32)


# ---------------------------------------------------------------------------
# Quantisation (an encoding: steps written out in fp32, in this order)
# ---------------------------------------------------------------------------

def tensor_global(x32):
    """Decode multiplier g = amax / 2688 (fp32 division); 1.0 for a zero tensor."""
    x32 = np.asarray(x32, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    if amax > 0:
        return np.float32(amax / np.float32(QUANT_RANGE))
    return np.float32(1.0)


def quantize(x, g=None):
    """Quantise a real matrix x[N, K] (K % 16 == 0) to NVFP4.

    Steps, each an fp32 operation rounded to nearest-even:
      1. g = amax(|x|) / 2688 over the whole tensor (or the given g).
      2. per 16-block b:  s = e4m3_rne_sat( amax_b / (6 * g) ),
         denom = e4m3(s) * g.
      3. per element:     code = e2m1_rne_sat( x * (1 / denom) ),
         code 0 for every element of a block whose denom is 0.
      4. pack two codes per byte, element 2i in the low nibble.
    Returns (codes [N, K/2] u8, scales [N, K/16] u8, g float32).
    """
    x32 = np.asarray(x, dtype=np.float32)
    if x32.ndim != 2 or x32.shape[1] % 16:
        raise ValueError("x must be [N, K] with K % 16 == 0")
    if not np.all(np.isfinite(x32)):
        raise ValueError("non-finite input")
    g = tensor_global(x32) if g is None else np.float32(g)
    if not (g > 0 and np.isfinite(g)):
        raise ValueError("global scale must be positive and finite")
    n, k = x32.shape
    blocks = x32.reshape(n, k // 16, 16)
    amax_b = np.max(np.abs(blocks), axis=2)                     # exact
    s_f = (amax_b / (np.float32(E2M1_MAX) * g)).astype(np.float32)
    s_code = e4m3_rne_saturate(s_f)
    s_dec = decode_e4m3(s_code).astype(np.float32)               # exact
    denom = (s_dec * g).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(denom > 0, np.float32(1.0) / np.where(denom > 0, denom, 1), 0)
    inv = inv.astype(np.float32)
    v = (blocks * inv[:, :, None]).astype(np.float32)
    codes = e2m1_rne_saturate(v)
    # a zero denominator keeps every code of its block at +0
    codes = np.where((denom > 0)[:, :, None], codes, 0).astype(np.uint8)
    return pack_nibbles(codes.reshape(n, k)), s_code.reshape(n, k // 16), np.float32(g)


# ---------------------------------------------------------------------------
# bf16 rounding (round-to-nearest-even, straight from fp64)
# ---------------------------------------------------------------------------

def bf16_rne(v):
    """Nearest bf16 value of each fp64 v, ties to even; values stay fp64.

    bf16 keeps 8 significant bits and fp32's exponent range; below 2**-126
    the spacing is fixed at 2**-133 (bf16 subnormals).
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite value")
    _, e = np.frexp(v)                        # v = f * 2**e, 0.5 <= |f| < 1
    e = np.maximum(e, -125)
    q = np.exp2(e - 8.0)                      # spacing of bf16 at v
    r = np.rint(v / q) * q                    # rint is half-to-even
    if np.any(np.abs(r) > 3.3895313892515355e38):
        raise OverflowError("bf16 overflow")
    return r


# ---------------------------------------------------------------------------
# Linear maps
# ---------------------------------------------------------------------------

def linear(x, codes, scales, g, act_quant=False, act_global=None):
    """y = x . deq(W)^T in fp64 for W [N, K] NVFP4 and x [M, K].

    With act_quant (W4A4) x is first replaced by deq(quantize(x)) with one
    tensor scale over all of x (computed, or act_global when given).
    Returns (y fp64 [M, N], the activation global used or None).
    """
    x64 = np.asarray(x, dtype=np.float64)
    a_g = None
    if act_quant:
        xc, xs, a_g = quantize(np.asarray(x, dtype=np.float32), act_global)
        x64 = dequantize(xc, xs, a_g)
    d = block_values(codes, scales)
    y = (x64 @ d.T) * np.float64(np.float32(g))
    return y, a_g


def silu(z):
    """z * sigmoid(z) in fp64."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


# ---------------------------------------------------------------------------
# Routing
# ---------------------------------------------------------------------------

def router_logits(x, r, bias=None):
    """Router logits l[t][e] = sum_h x[t][h] r[e][h] (+ bias[e]) in fp64.

    x [T, H] and r [E, H] hold bf16 values (the router stays BF16 beside the
    NVFP4 routed experts: Qwen3.8-Flash-Next-NVFP4-SSD-Stream model card,
    "What this model is"); bias is fp32 [E] or None.
    """
    lg = np.asarray(x, dtype=np.float64) @ np.asarray(r, dtype=np.float64).T
    if bias is not None:
        lg = lg + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return lg


def route_topk(logits, k, renormalize=True):
    """Top-k experts per token from fp32 logits [T, E].

    Experts are ordered by descending logit; equal logits go to the lower
    expert index.  Weights: with renormalize, exp(l_j - l_max) over the k
    chosen, divided by their sum (top-k of softmax, renormalised: the full
    softmax denominator cancels); without, softmax over all E.  fp64.
    Returns (ids [T, k] int32, weights [T, k] float64).
    """
    l32 = np.asarray(logits, dtype=np.float32)
    if not np.all(np.isfinite(l32)):
        raise ValueError("non-finite logits")
    t, e = l32.shape
    if not (1 <= k <= e):
        raise ValueError("need 1 <= k <= E")
    ids = np.empty((t, k), dtype=np.int32)
    w = np.empty((t, k), dtype=np.float64)
    for i in range(t):
        order = sorted(range(e), key=lambda j: (-float(l32[i, j]), j))
        ids[i] = order[:k]
        l64 = l32[i].astype(np.float64)
        ex = np.exp(l64 - l64.max())
        denom = ex[ids[i]].sum() if renormalize else ex.sum()
        w[i] = ex[ids[i]] / denom
    return ids, w


def permute(ids, num_experts):
    """Expert-sorted list of pairs.

    A pair is p = t*k + j (token t, slot j).  Pairs are ordered by expert,
    then by token (a stable counting sort).  A pair whose id lies outside
    0..E-1 is dropped: it takes no position, offsets[E] counts the kept
    pairs, and the positions after them hold -1.  Returns
    (offsets [E+1] int32 with offsets[e]..offsets[e+1] the rows of expert
    e, sorted_pairs [T*k] int32).
    """
    ids = np.asarray(ids)
    t, k = ids.shape
    counts = np.zeros(num_experts, dtype=np.int64)
    for e in ids.reshape(-1):
        if 0 <= e < num_experts:
            counts[e] += 1
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    fill = offsets[:-1].copy()
    sorted_pairs = np.full(t * k, -1, dtype=np.int64)
    for p in range(t * k):                     # p ascending => t ascending
        e = ids[p // k, p % k]
        if not 0 <= e < num_experts:
            continue
        sorted_pairs[fill[e]] = p
        fill[e] += 1
    return offsets.astype(np.int32), sorted_pairs.astype(np.int32)


# ---------------------------------------------------------------------------
# Expert FFN
# ---------------------------------------------------------------------------

class ExpertWeights:
    """Stacked NVFP4 expert weights (numpy arrays, one entry per expert).

    gate/up codes [E, I, H/2], scales [E, I, H/16]; down codes [E, H, I/2],
    scales [E, H, I/16]; globals [E] float32 each.
    """

    def __init__(self, gate_codes, gate_scales, gate_global,
                 up_codes, up_scales, up_global,
                 down_codes, down_scales, down_global):
        self.gate_codes, self.gate_scales = gate_codes, gate_scales
        self.up_codes, self.up_scales = up_codes, up_scales
        self.down_codes, self.down_scales = down_codes, down_scales
        self.gate_global = np.asarray(gate_global, dtype=np.float32)
        self.up_global = np.asarray(up_global, dtype=np.float32)
        self.down_global = np.asarray(down_global, dtype=np.float32)


def expert_h(x_rows, w, e):
    """bf16_rne( silu(g_gate * x D_gate^T) * (g_up * x D_up^T) ) for expert e."""
    dg = block_values(w.gate_codes[e], w.gate_scales[e])
    du = block_values(w.up_codes[e], w.up_scales[e])
    gate = (x_rows @ dg.T) * np.float64(w.gate_global[e])
    up = (x_rows @ du.T) * np.float64(w.up_global[e])
    return bf16_rne(silu(gate) * up)


def expert_h_fp32(xv_rows, g_x, w, e):
    """h for expert e with the gate and up values formed in fp32, for where an
    h value decides an integer (its bf16 rounding and, in W4A4, its NVFP4
    code) and both sides must take that decision in the same precision.

    Reading: the FFN accumulates in fp32, so each value is an fp32 operation
    rounded to nearest-even, in the order the definition is written:
      S = fl32(exact x_v . D^T)  (x_v: the unscaled operand, e2m1*e4m3 blocks
          of the quantised x, or the bf16 x itself; every product is exact),
      G = fl32(S * fl32(g_gate * g_x)), U likewise with g_up (g_x = 1 for a
          bf16 x),
      h = bf16_rne( fl32( fl32(G / fl32(1 + fl32(exp(-G)))) * U ) ),
    exp itself correctly rounded from fp64.
    """
    f32 = np.float32
    gx = f32(1.0) if g_x is None else f32(g_x)
    dg = block_values(w.gate_codes[e], w.gate_scales[e])
    du = block_values(w.up_codes[e], w.up_scales[e])
    with np.errstate(over="ignore"):
        s_g = (xv_rows @ dg.T).astype(f32)
        s_u = (xv_rows @ du.T).astype(f32)
        gate = s_g * (f32(w.gate_global[e]) * gx)
        up = s_u * (f32(w.up_global[e]) * gx)
        ex = np.exp(-gate.astype(np.float64)).astype(f32)
        h32 = (gate / (f32(1.0) + ex)) * up
    return bf16_rne(h32.astype(np.float64))


# ---------------------------------------------------------------------------
# Where h decides an integer: the fp32 error of h and the valid roundings
# ---------------------------------------------------------------------------

U32 = 2.0 ** -24   # unit roundoff of fp32


def bf16_bracket(v):
    """The bf16 values lo <= v <= hi around each fp64 v (lo == hi when v is a
    bf16 value).  bf16 keeps 8 significant bits: in the binade
    [2**(e-1), 2**e) the spacing is 2**(e-8)."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    q = np.exp2(np.maximum(e, -125) - 8.0)
    lo = np.floor(v / q) * q
    hi = np.where(lo == v, lo, lo + q)
    return lo, hi


def expert_h_bound(xv_rows, g_x, w, e, lam=8.0):
    """h of expert e before its bf16 rounding, in fp64, and a bound on how far
    an fp32 evaluation of the same definition can land from it.

    xv_rows are the unscaled activation operand (the e2m1 * e4m3 blocks of
    the quantised x with g_x, or the bf16 x itself with g_x = None); every
    product p_i = xv_i * D_i is exact in fp32.  Reading of "within a few
    fp32 ulps" for a K-term fp32 sum S = sum p_i: the rounding errors of
    the additions behave as independent and the partial sums as random
    walks (the products have random signs), so in any summation order
    |fl32(S) - S| <= lam * u * sqrt(K) * ||p||_2  (u = 2**-24; with errors
    uniform in [-u, u] relative to each partial sum the standard deviation
    is about 0.4 u sqrt(K) ||p||_2, so lam = 8 keeps twenty of them; sums
    of these few-bit products are often exact, so real errors sit far
    lower).  The scale products and the SiLU * up step add a few more
    roundings:
      dG = |g| dS_g + 2 u |G|,  dU likewise,
      dh = |silu'(G) U| dG + |silu(G)| dU + 8 u |h|.
    Returns (h64 [n, I], dh [n, I])."""
    xv = np.asarray(xv_rows, dtype=np.float64)
    gx = 1.0 if g_x is None else float(np.float32(g_x))
    dg = block_values(w.gate_codes[e], w.gate_scales[e])
    du = block_values(w.up_codes[e], w.up_scales[e])
    k = dg.shape[1]
    cg = float(np.float32(w.gate_global[e])) * gx
    cu = float(np.float32(w.up_global[e])) * gx
    x2 = xv * xv
    gate = (xv @ dg.T) * cg
    up = (xv @ du.T) * cu
    d_sg = lam * np.sqrt(k) * U32 * np.sqrt(x2 @ (dg * dg).T)
    d_su = lam * np.sqrt(k) * U32 * np.sqrt(x2 @ (du * du).T)
    d_gate = abs(cg) * d_sg + 2 * U32 * np.abs(gate)
    d_up = abs(cu) * d_su + 2 * U32 * np.abs(up)
    sig = 1.0 / (1.0 + np.exp(-gate))
    h64 = gate * sig * up
    dsilu = sig * (1.0 + gate * (1.0 - sig))
    dh = np.abs(dsilu * up) * d_gate + np.abs(gate * sig) * d_up + 8 * U32 * np.abs(h64)
    return h64, dh


def check_h_choices(h64, dh, h_dev):
    """Which bf16 values of h are valid results (the several-results-correct
    reading for where h decides an integer).  Where h64 lies further than dh
    from the midpoint of its two bf16 neighbours, only bf16_rne(h64) is
    valid; within dh of it, either neighbour is (an fp32 evaluation can land
    on either side).  Returns (ok, flagged, flips): boolean arrays of the
    shape of h64 (ok: h_dev is a valid value; flagged: both neighbours are
    valid there; flips: h_dev differs from bf16_rne(h64))."""
    h64 = np.asarray(h64, dtype=np.float64)
    h_dev = np.asarray(h_dev, dtype=np.float64)
    lo, hi = bf16_bracket(h64)
    rne = bf16_rne(h64)
    flagged = (lo != hi) & (np.abs(h64 - 0.5 * (lo + hi)) <= np.asarray(dh, dtype=np.float64))
    ok = (h_dev == rne) | (flagged & ((h_dev == lo) | (h_dev == hi)))
    return ok, flagged, h_dev != rne


def expert_down(h_rows, w, e):
    """g_down * h D_down^T for expert e (fp64)."""
    dd = block_values(w.down_codes[e], w.down_scales[e])
    return (h_rows @ dd.T) * np.float64(w.down_global[e])


def moe_ffn(x, ids, weights, w, act_quant=False, act_globals=None,
            tokens=None, h_fp32=False, h_given=None, with_bound=False):
    """Routed-expert FFN, fp64.

    y_t = sum_j weights[t, j] * down_e( h ),  e = ids[t, j], where
    h = bf16_rne(silu(gate_e(x_t)) * up_e(x_t)).  The experts are visited
    one at a time, so only one expert is ever dense in memory.  A pair whose
    id lies outside 0..E-1 is dropped: it contributes nothing to y (a token
    without kept pairs gets 0) and takes no part in any tensor scale.

    W4A4 (act_quant): x is replaced by deq(quantize(x)) with one tensor scale
    over all T rows, and h (over all kept pairs) by deq(quantize(h)) with one
    tensor scale over those pairs, before the down projection.
    act_globals = (g_x, g_h) fixes those scales instead of computing them.
    tokens: compute only these output rows (W4A16, or W4A4 with both
    act_globals given, where the rows are independent).
    h_fp32: form h with expert_h_fp32 (fp32 gate/up values) instead of fp64;
    everything after h stays as above.
    h_given: bf16 values [len(tokens), k, I] to use as h of the kept pairs
    (a device's valid choices where h decides an integer; everything after h
    is computed from them as above).
    with_bound: also return info["h64"] (h before its bf16 rounding) and
    info["h_bound"] (expert_h_bound's dh) for the kept pairs.
    Returns (y fp64 [T or len(tokens), H], info dict; info["h_bf16"] is h
    before its W4A4 quantisation, info["h"] the h the down projection used,
    info["kept"] the [n, k] mask of kept pairs).
    """
    x32 = np.asarray(x, dtype=np.float32)
    ids = np.asarray(ids)
    weights = np.asarray(weights, dtype=np.float64)
    t_all, hdim = x32.shape
    k = ids.shape[1]
    n_exp = w.gate_codes.shape[0]
    idim = w.gate_codes.shape[1]
    info = {}
    if tokens is None:
        tokens = np.arange(t_all)
    tokens = np.asarray(tokens, dtype=np.int64)
    if act_quant and (act_globals is None or act_globals[1] is None) \
            and len(tokens) != t_all:
        raise ValueError("online h scale needs every token")

    if act_quant:
        g_x = None if act_globals is None else act_globals[0]
        xc, xs, g_x = quantize(x32, g_x)
        x64 = dequantize(xc, xs, g_x)
        info["g_x"] = g_x
        xv, xv_g = block_values(xc, xs), g_x
    else:
        x64 = x32.astype(np.float64)
        xv, xv_g = x64, None

    # h for every requested (token, slot) of a kept pair, expert by expert
    sel_ids = ids[tokens]                                    # [n, k]
    kept = (sel_ids >= 0) & (sel_ids < n_exp)
    experts = np.unique(sel_ids[kept])
    h = np.zeros((len(tokens), k, idim), dtype=np.float64)
    if with_bound:
        h64 = np.zeros_like(h)
        hb = np.zeros_like(h)
    for e in experts:
        rows, slots = np.nonzero(sel_ids == e)
        if with_bound:
            h64[rows, slots], hb[rows, slots] = expert_h_bound(xv[tokens[rows]], xv_g, w, e)
        if h_given is not None:
            continue
        h[rows, slots] = (expert_h_fp32(xv[tokens[rows]], xv_g, w, e) if h_fp32
                          else expert_h(x64[tokens[rows]], w, e))
    if h_given is not None:
        h = np.where(kept[:, :, None], np.asarray(h_given, dtype=np.float64), 0.0)
    if with_bound:
        info["h64"], info["h_bound"] = h64, hb
    info["h_bf16"] = h.copy()

    if act_quant:
        g_h = None if act_globals is None else act_globals[1]
        flat = h[kept]                                       # [kept pairs, I]
        if flat.shape[0]:
            hc, hs, g_h = quantize(flat.astype(np.float32), g_h)
            h[kept] = dequantize(hc, hs, g_h)
        info["g_h"] = np.float32(1.0) if g_h is None else np.float32(g_h)

    y = np.zeros((len(tokens), hdim), dtype=np.float64)
    for e in experts:
        rows, slots = np.nonzero(sel_ids == e)
        contrib = expert_down(h[rows, slots], w, e)
        np.add.at(y, rows, contrib * weights[tokens[rows], slots][:, None])
    info["h"] = h
    info["kept"] = kept
    return y, info


def shared_expert(x, w_gate, w_up, w_down, y_in=None):
    """The BF16 shared expert (Qwen3.8-Flash-Next-NVFP4-SSD-Stream model card,
    "What this model is": shared experts stay BF16), fp64:
    h = bf16_rne(silu(x Wg^T) * (x Wu^T)), y = h Wd^T, plus y_in when given.
    x [T, H], w_gate / w_up [I, H], w_down [H, I] hold bf16 values.
    """
    x64 = np.asarray(x, dtype=np.float64)
    gate = x64 @ np.asarray(w_gate, dtype=np.float64).T
    up = x64 @ np.asarray(w_up, dtype=np.float64).T
    h = bf16_rne(silu(gate) * up)
    y = h @ np.asarray(w_down, dtype=np.float64).T
    return y if y_in is None else np.asarray(y_in, dtype=np.float64) + y


def dense_mlp(x, gate, up, down):
    """Dense gated MLP y = down(silu(gate x) * up x) over NVFP4 matrices.

    gate, up, down are (codes, scales, g) triples; this is the expert FFN
    with one expert, one slot and routing weight 1.
    """
    w = ExpertWeights(gate[0][None], gate[1][None], [gate[2]],
                      up[0][None], up[1][None], [up[2]],
                      down[0][None], down[1][None], [down[2]])
    t = np.asarray(x).shape[0]
    ids = np.zeros((t, 1), dtype=np.int32)
    y, _ = moe_ffn(x, ids, np.ones((t, 1)), w)
    return y


# ---------------------------------------------------------------------------
# Expert paging: the slot plan of a bounded expert pool
# ---------------------------------------------------------------------------

class SlotState:
    """A pool of S expert slots in front of E experts (Eider page, "Why Eider
    exists": selected experts resident in bounded page pools, the rest paged
    in).  slot_of[e] is expert e's slot or -1; expert_of[s] is slot s's
    expert or -1; last_use[s] is the stamp of the last step that used slot s;
    hand is the clock hand (the slot the next search starts from)."""

    def __init__(self, E, S):
        self.E, self.S = E, S
        self.slot_of = [-1] * E
        self.expert_of = [-1] * S
        self.last_use = [0] * S
        self.hand = 0

    def copy(self):
        c = SlotState(self.E, self.S)
        c.slot_of, c.expert_of = list(self.slot_of), list(self.expert_of)
        c.last_use, c.hand = list(self.last_use), self.hand
        return c


def expert_slot_plan(state, ids, step, protect_from, max_fetch=None):
    """One step's slot plan (the pages give no policy; this is the reading
    the library implements, a clock-order replacement):

    1. The needed experts are the distinct ids of the step (ids outside
       0..E-1 are ignored).  A needed expert that is resident keeps its slot
       and the slot's stamp becomes `step`.
    2. The missing needed experts, in ascending expert order, take the free
       slots met walking from the hand: a slot is free when it is empty, or
       when its expert is not needed now and its stamp is below
       protect_from (a step whose FFN may still run passes its own stamp).
       Missing expert i takes free slot i, evicting that slot's expert, and
       the slot gets the stamp `step`; the hand moves just past the last
       slot taken.
    3. If the free slots are fewer than the missing experts, or the missing
       experts are more than max_fetch (the most one step's fetch copies;
       None: no limit), nothing of step 2 happens and n_fetch is -1.

    Returns (slot_ids [T, k] int32: each pair's slot, or -1 for an ignored
    id or an expert left without a slot, so that later steps drop the pair;
    the fetch list [(expert, slot)]; n_fetch).  `state` is updated in place."""
    E, S = state.E, state.S
    ids = np.asarray(ids)
    needed = sorted({int(e) for e in ids.ravel() if 0 <= e < E})
    missing = []
    for e in needed:
        s = state.slot_of[e]
        if s >= 0:
            state.last_use[s] = step
        else:
            missing.append(e)
    needed_set = set(needed)
    free = []
    for r in range(S):
        s = (state.hand + r) % S
        e = state.expert_of[s]
        if e < 0 or (e not in needed_set and state.last_use[s] < protect_from):
            free.append(s)
    fetch = []
    if len(missing) <= len(free) and (max_fetch is None or len(missing) <= max_fetch):
        for e, s in zip(missing, free):
            old = state.expert_of[s]
            if old >= 0:
                state.slot_of[old] = -1
            state.slot_of[e], state.expert_of[s], state.last_use[s] = s, e, step
            fetch.append((e, s))
        if missing:
            state.hand = (free[len(missing) - 1] + 1) % S
        n_fetch = len(missing)
    else:
        n_fetch = -1
    slot_ids = np.full(ids.shape, -1, np.int32)
    for idx, e in np.ndenumerate(ids):
        if 0 <= e < E and state.slot_of[int(e)] >= 0:
            slot_ids[idx] = state.slot_of[int(e)]
    return slot_ids, fetch, n_fetch
