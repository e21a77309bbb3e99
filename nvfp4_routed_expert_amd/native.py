"""Thin Python binding of libnvfp4moe.so (include/nvfp4moe.h).

Argument marshalling only: PyTorch allocates device memory and supplies the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library is missing or cannot be
loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnvfp4moe.so")

OK = 0
DT_BF16, DT_F32 = 0, 1
GLOBAL_COMPUTE, GLOBAL_GIVEN = 0, 1
W4A16, W4A4 = 0, 1

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t


class NVFP4Error(RuntimeError):
    def __init__(self, status, text, detail):
        super().__init__(f"{text} ({status}): {detail}")
        self.status = status


class Matrix(ctypes.Structure):
    _fields_ = [("codes", _vp), ("scales", _vp), ("global_scale", _vp),
                ("rows", _i64), ("cols", _i64)]


class ExpertWeightsC(ctypes.Structure):
    _fields_ = [("gate_codes", _vp), ("up_codes", _vp), ("down_codes", _vp),
                ("gate_scales", _vp), ("up_scales", _vp), ("down_scales", _vp),
                ("gate_global", _vp), ("up_global", _vp), ("down_global", _vp)]


_LIB = None


def lib():
    """Load the HIP library (once).  Raises if it is not built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m nvfp4_routed_expert_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        sigs = {
            "nvfp4_quantize": (_i32, [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _i32,
                                      _vp, _sz, _vp]),
            "nvfp4_quantize_workspace_size": (_sz, [_i64, _i64]),
            "nvfp4_dequantize": (_i32, [ctypes.POINTER(Matrix), _vp, _vp]),
            "nvfp4_linear": (_i32, [_vp, _i64, ctypes.POINTER(Matrix), _i32, _i32, _vp, _vp,
                                    _i32, _vp, _sz, _vp]),
            "nvfp4_linear_workspace_size": (_sz, [_i64, _i64, _i64, _i32]),
            "moe_route_topk": (_i32, [_vp, _i64, _i32, _i32, ctypes.c_int, _vp, _vp, _vp, _vp,
                                      _vp, _sz, _vp]),
            "moe_route_topk_workspace_size": (_sz, [_i64, _i32, _i32]),
            "moe_route_workspace_init": (_i32, [_vp, _sz, _vp]),
            "moe_router_topk": (_i32, [_vp, _i64, _i64, _vp, _vp, _i32, _i32, ctypes.c_int, _vp,
                                       _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
            "moe_router_topk_workspace_size": (_sz, [_i64, _i64, _i32, _i32]),
            "moe_shared_expert_ffn": (_i32, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, ctypes.c_int,
                                             _vp, _i32, _vp, _sz, _vp]),
            "moe_shared_expert_ffn_workspace_size": (_sz, [_i64, _i64, _i64]),
            "moe_expert_cache_init": (_i32, [_vp, _i32, _vp, _vp, _vp, _i32, _vp]),
            "moe_expert_cache_plan": (_i32, [_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                             ctypes.c_uint32, ctypes.c_uint32, _i32, _vp, _vp,
                                             _vp, _vp]),
            "moe_expert_cache_fetch": (_i32, [ctypes.POINTER(ExpertWeightsC),
                                              ctypes.POINTER(ExpertWeightsC), _i64, _i64, _vp,
                                              _vp, _i32, _vp]),
            "moe_permute_pairs": (_i32, [_vp, _i64, _i32, _i32, _vp, _vp, _vp]),
            "moe_grouped_nvfp4_ffn": (_i32, [_vp, _i64, _i64, _i64, _i32, _i32, _vp, _vp, _vp,
                                             _vp, ctypes.POINTER(ExpertWeightsC), _i32, _i32,
                                             _vp, _vp, _i32, _vp, _sz, _vp]),
            "moe_grouped_nvfp4_ffn_workspace_size": (_sz, [_i64, _i64, _i64, _i32, _i32, _i32]),
            "moe_route_ffn_decode": (_i32, [_vp, _vp, _i64, _i64, _i64, _i32, _i32, ctypes.c_int,
                                            _vp, _vp, _vp, _vp, ctypes.POINTER(ExpertWeightsC),
                                            _vp, _i32, _vp, _sz, _vp]),
            "moe_route_ffn_decode_workspace_size": (_sz, [_i64, _i64, _i64, _i32, _i32]),
            "moe_grouped_nvfp4_ffn_static": (_i32, [_vp, _i64, _i64, _i64, _i32, _i32, _vp, _vp,
                                                    _vp, _vp, ctypes.POINTER(ExpertWeightsC),
                                                    _i32, _i32, _vp, _vp, _i32, _vp]),
            "moe_grouped_nvfp4_ffn_static_max_bytes": (_sz, []),
            "moe_grouped_nvfp4_ffn_debug_h": (ctypes.c_int, [_i64, _i64, _i64, _i32, _i32, _i32,
                                                             _i32, ctypes.POINTER(_sz),
                                                             ctypes.POINTER(_sz)]),
            "nvfp4_set_ffn_stage_events": (None, [_vp]),
            "nvfp4_set_ffn_separate_h_quant": (None, [ctypes.c_int]),
            "nvfp4_read_probe": (_i32, [_vp, _sz, _vp, _vp]),
            "nvfp4_status_string": (ctypes.c_char_p, [_i32]),
            "nvfp4_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


FFN_STAGES = ("plan", "x_prep", "gate_up", "h_prep", "down", "combine")


def exported_symbols():
    return ["nvfp4_quantize", "nvfp4_quantize_workspace_size", "nvfp4_dequantize",
            "nvfp4_linear", "nvfp4_linear_workspace_size", "moe_route_topk",
            "moe_route_topk_workspace_size", "moe_route_workspace_init", "moe_router_topk",
            "moe_router_topk_workspace_size",
            "moe_shared_expert_ffn", "moe_shared_expert_ffn_workspace_size",
            "moe_expert_cache_init", "moe_expert_cache_plan", "moe_expert_cache_fetch",
            "moe_permute_pairs",
            "moe_grouped_nvfp4_ffn",
            "moe_grouped_nvfp4_ffn_workspace_size", "moe_grouped_nvfp4_ffn_debug_h",
            "moe_route_ffn_decode", "moe_route_ffn_decode_workspace_size",
            "moe_grouped_nvfp4_ffn_static", "moe_grouped_nvfp4_ffn_static_max_bytes",
            "nvfp4_set_ffn_stage_events",
            "nvfp4_set_ffn_separate_h_quant", "nvfp4_read_probe",
            "nvfp4_status_string", "nvfp4_last_error"]


def _check(status):
    if status != OK:
        L = lib()
        raise NVFP4Error(status, L.nvfp4_status_string(status).decode(),
                         L.nvfp4_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _workspace(nbytes, device, workspace=None):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace needs {nbytes} bytes")
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _dt(dtype):
    if dtype == torch.bfloat16:
        return DT_BF16
    if dtype == torch.float32:
        return DT_F32
    raise TypeError(f"unsupported dtype {dtype}")


# ---------------------------------------------------------------------------


def nvfp4_quantize(x, global_scale=None, workspace=None, out=None):
    """Quantise x [rows, cols] (bf16/f32, cuda) to NVFP4.

    global_scale: None computes g = amax/2688; a 1-element fp32 cuda tensor
    is used as the given decode scale.  Returns (codes, scales, g).
    """
    rows, cols = x.shape
    dev = x.device
    if out is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
    else:
        codes, scales = out
    if global_scale is None:
        g = torch.empty(1, dtype=torch.float32, device=dev)
        mode = GLOBAL_COMPUTE
    else:
        g, mode = global_scale, GLOBAL_GIVEN
    L = lib()
    nbytes = L.nvfp4_quantize_workspace_size(rows, cols)
    ws = _workspace(nbytes, dev, workspace)
    _check(L.nvfp4_quantize(_ptr(x), _dt(x.dtype), rows, cols, x.stride(0), _ptr(codes),
                            _ptr(scales), _ptr(g), mode, _ptr(ws), ws.numel(), _stream()))
    return codes, scales, g


def nvfp4_dequantize(codes, scales, g):
    rows, half = codes.shape
    out = torch.empty((rows, half * 2), dtype=torch.float32, device=codes.device)
    m = Matrix(codes.data_ptr(), scales.data_ptr(), g.data_ptr(), rows, half * 2)
    _check(lib().nvfp4_dequantize(ctypes.byref(m), _ptr(out), _stream()))
    return out


def nvfp4_linear(x, codes, scales, g, act=W4A16, act_global=None,
                 out_dtype=torch.bfloat16, workspace=None, out=None):
    """y [M, N] = x [M, K] . deq(W [N, K])^T.  W4A4 quantises x first.

    act_global (W4A4): None -> computed (returned); a tensor -> given.
    Returns (y, act_global or None).
    """
    M, K = x.shape
    N = codes.shape[0]
    dev = x.device
    y = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=dev)
    mode = GLOBAL_COMPUTE
    ag = None
    if act == W4A4:
        if act_global is None:
            ag = torch.empty(1, dtype=torch.float32, device=dev)
        else:
            ag, mode = act_global, GLOBAL_GIVEN
    L = lib()
    ws = _workspace(L.nvfp4_linear_workspace_size(M, N, K, act), dev, workspace)
    m = Matrix(codes.data_ptr(), scales.data_ptr(), g.data_ptr(), N, K)
    _check(L.nvfp4_linear(_ptr(x), M, ctypes.byref(m), act, mode, _ptr(ag), _ptr(y),
                          _dt(y.dtype), _ptr(ws), ws.numel(), _stream()))
    return y, ag


def _init_route_workspace(ws):
    _check(lib().moe_route_workspace_init(_ptr(ws), ws.numel(), _stream()))
    return ws


def route_workspace(T, E, k, device):
    """A routing workspace made ready by moe_route_workspace_init (its ticket
    word zeroed on the current stream); every call leaves it ready again, so
    one workspace serves successive (not overlapping) calls on a stream."""
    ws = torch.empty(max(lib().moe_route_topk_workspace_size(T, E, k), 4), dtype=torch.uint8,
                     device=device)
    return _init_route_workspace(ws)


def moe_route_topk(logits, k, renormalize=True, out=None, workspace=None, permute=True):
    """Returns (topk_ids [T,k] i32, topk_weights [T,k] f32, expert_offsets [E+1] i32,
    sorted_pairs [T*k] i32).  workspace: from route_workspace (a fresh zeroed
    one is made when omitted).  permute=False: the top-k alone (offsets and
    pairs returned as None; moe_permute_pairs makes them)."""
    T, E = logits.shape
    dev = logits.device
    if out is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        off = torch.empty(E + 1, dtype=torch.int32, device=dev) if permute else None
        pairs = torch.empty(T * k, dtype=torch.int32, device=dev) if permute else None
    else:
        ids, w, off, pairs = out
        if not permute:
            off = pairs = None
    L = lib()
    nbytes = L.moe_route_topk_workspace_size(T, E, k)
    if not permute:
        ws, nbytes = None, 0
    else:
        ws = _workspace(nbytes, dev, workspace) if workspace is not None else \
            route_workspace(T, E, k, dev)
    _check(L.moe_route_topk(_ptr(logits), T, E, k, int(bool(renormalize)), _ptr(ids), _ptr(w),
                            _ptr(off), _ptr(pairs), _ptr(ws), nbytes, _stream()))
    return ids, w, off, pairs


def router_workspace(T, H, E, k, device):
    """A zeroed workspace for moe_router_topk (left with its first word zero
    by every call, as for the routing workspace)."""
    ws = torch.empty(max(lib().moe_router_topk_workspace_size(T, H, E, k), 4),
                     dtype=torch.uint8, device=device)
    return _init_route_workspace(ws)


def moe_router_topk(x, router_w, k, renormalize=True, bias=None, want_logits=False, out=None,
                    workspace=None):
    """Router logits x [T,H] bf16 . router_w [E,H]^T bf16 (+ bias [E] f32), then
    the same top-k and permutation as moe_route_topk.  Returns (topk_ids,
    topk_weights, expert_offsets, sorted_pairs, logits or None)."""
    T, H = x.shape
    E = router_w.shape[0]
    dev = x.device
    if out is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        off = torch.empty(E + 1, dtype=torch.int32, device=dev)
        pairs = torch.empty(T * k, dtype=torch.int32, device=dev)
    else:
        ids, w, off, pairs = out
    logits = torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None
    L = lib()
    nbytes = L.moe_router_topk_workspace_size(T, H, E, k)
    ws = _workspace(nbytes, dev, workspace) if workspace is not None else \
        router_workspace(T, H, E, k, dev)
    _check(L.moe_router_topk(_ptr(x), T, H, _ptr(router_w), _ptr(bias), E, k,
                             int(bool(renormalize)), _ptr(logits), _ptr(ids), _ptr(w), _ptr(off),
                             _ptr(pairs), _ptr(ws), nbytes, _stream()))
    return ids, w, off, pairs, logits


def moe_shared_expert_ffn(x, w_gate, w_up, w_down, y=None, accumulate=False,
                          out_dtype=torch.bfloat16, workspace=None):
    """BF16 shared expert: y (+)= down(silu(x Wg^T) * (x Wu^T)).  x [T,H] bf16,
    w_gate / w_up [I,H] bf16, w_down [H,I] bf16.  y: the output (read first
    when accumulate), else a new tensor of out_dtype.  Returns y."""
    T, H = x.shape
    I = w_gate.shape[0]
    dev = x.device
    if y is None:
        if accumulate:
            raise ValueError("accumulate needs y")
        y = torch.empty((T, H), dtype=out_dtype, device=dev)
    L = lib()
    ws = _workspace(L.moe_shared_expert_ffn_workspace_size(T, H, I), dev, workspace)
    _check(L.moe_shared_expert_ffn(_ptr(x), T, H, I, _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                   int(bool(accumulate)), _ptr(y), _dt(y.dtype), _ptr(ws),
                                   ws.numel(), _stream()))
    return y


class ExpertWeights:
    """Device tensors of E stacked NVFP4 experts (gate/up [E,I,H], down [E,H,I])."""

    def __init__(self, gate_codes, gate_scales, gate_global, up_codes, up_scales,
                 up_global, down_codes, down_scales, down_global):
        self.gate_codes, self.gate_scales, self.gate_global = gate_codes, gate_scales, gate_global
        self.up_codes, self.up_scales, self.up_global = up_codes, up_scales, up_global
        self.down_codes, self.down_scales, self.down_global = down_codes, down_scales, down_global

    @property
    def num_experts(self):
        return self.gate_codes.shape[0]

    @property
    def intermediate(self):
        return self.gate_codes.shape[1]

    @property
    def hidden(self):
        return self.down_codes.shape[1]

    def c_struct(self):
        return ExpertWeightsC(*(t.data_ptr() for t in (
            self.gate_codes, self.up_codes, self.down_codes, self.gate_scales,
            self.up_scales, self.down_scales, self.gate_global, self.up_global,
            self.down_global)))


def moe_permute_pairs(topk_ids, num_experts, out=None):
    """Expert offsets [E+1] and expert-sorted pairs [T*k] of given ids [T, k]."""
    T, k = topk_ids.shape
    dev = topk_ids.device
    if out is None:
        off = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
        pairs = torch.empty(T * k, dtype=torch.int32, device=dev)
    else:
        off, pairs = out
    _check(lib().moe_permute_pairs(_ptr(topk_ids), T, num_experts, k, _ptr(off), _ptr(pairs),
                                   _stream()))
    return off, pairs


class ExpertCache:
    """Expert paging: host_weights (an ExpertWeights of E experts whose tensors
    are in pinned host memory) behind a device pool of `slots` experts.
    plan_and_fetch(ids) maps a step's expert ids to slots and copies the
    missing experts into the pool (on the current stream, no host round
    trip); the FFN then runs on `pool` with the slot ids and slots experts."""

    def __init__(self, host_weights, slots, device):
        self.host = host_weights
        self.E, self.S = host_weights.num_experts, slots
        self.H, self.I = host_weights.hidden, host_weights.intermediate
        ts = (host_weights.gate_codes, host_weights.gate_scales, host_weights.gate_global,
              host_weights.up_codes, host_weights.up_scales, host_weights.up_global,
              host_weights.down_codes, host_weights.down_scales, host_weights.down_global)
        for t in ts:
            if not t.is_pinned():
                raise ValueError("host expert weights must be in pinned host memory")
        self.pool = ExpertWeights(*[torch.empty((slots,) + tuple(t.shape[1:]), dtype=t.dtype,
                                                device=device) for t in ts])
        i32 = dict(dtype=torch.int32, device=device)
        self.slot_of = torch.empty(self.E, **i32)
        self.expert_of = torch.empty(slots, **i32)
        self.last_use = torch.empty(slots, **i32)      # uint32 stamps
        self.hand = torch.empty(1, **i32)
        self.fetch = torch.empty(2 * slots, **i32)
        self.n_fetch = torch.zeros(1, **i32)
        self.step_no = 0
        self._host_c, self._pool_c = host_weights.c_struct(), self.pool.c_struct()
        _check(lib().moe_expert_cache_init(_ptr(self.slot_of), self.E, _ptr(self.expert_of),
                                           _ptr(self.last_use), _ptr(self.hand), slots,
                                           _stream()))

    def plan(self, topk_ids, protect_previous=False, slot_ids=None):
        """Slot ids [T, k] for this step's expert ids (the missing experts
        get slots; fetch() copies them).  protect_previous: keep the previous
        step's experts (its FFN may still be running)."""
        T, k = topk_ids.shape
        self.step_no += 1
        protect = self.step_no - 1 if protect_previous and self.step_no > 1 else self.step_no
        if slot_ids is None:
            slot_ids = torch.empty_like(topk_ids)
        _check(lib().moe_expert_cache_plan(_ptr(topk_ids), T, k, self.E, self.S,
                                           _ptr(self.slot_of), _ptr(self.expert_of),
                                           _ptr(self.last_use), _ptr(self.hand), self.step_no,
                                           protect, self.max_fetch(T * k), _ptr(slot_ids),
                                           _ptr(self.fetch), _ptr(self.n_fetch), _stream()))
        return slot_ids

    def max_fetch(self, pairs):
        """The most experts one step can fetch: min(slots, pairs)."""
        return min(self.S, pairs)

    def fetch_planned(self, pairs):
        """Copy the experts the last plan() listed (pairs = T * k of that step)."""
        _check(lib().moe_expert_cache_fetch(ctypes.byref(self._host_c),
                                            ctypes.byref(self._pool_c), self.H, self.I,
                                            _ptr(self.fetch), _ptr(self.n_fetch),
                                            self.max_fetch(pairs), _stream()))

    def plan_and_fetch(self, topk_ids, protect_previous=False, slot_ids=None):
        """plan() then fetch_planned(): slot ids [T, k], the pool filled."""
        slot_ids = self.plan(topk_ids, protect_previous, slot_ids)
        self.fetch_planned(topk_ids.numel())
        return slot_ids


def ffn_workspace_bytes(T, H, I, E, k, act=W4A16):
    return lib().moe_grouped_nvfp4_ffn_workspace_size(T, H, I, E, k, act)


def moe_grouped_nvfp4_ffn(x, weights: ExpertWeights, topk_ids, topk_weights, expert_offsets,
                          sorted_pairs, k, act=W4A16, act_globals=None,
                          out_dtype=torch.bfloat16, workspace=None, out=None):
    """Routed-expert gated FFN over moe_route_topk's outputs.  expert_offsets
    and sorted_pairs may both be None on the fused decode path (the pairs are
    then read in pair order).  Returns (y [T,H], act_globals or None)."""
    T, H = x.shape
    E, I = weights.num_experts, weights.intermediate
    dev = x.device
    y = out if out is not None else torch.empty((T, H), dtype=out_dtype, device=dev)
    mode = GLOBAL_COMPUTE
    ag = None
    if act == W4A4:
        if act_globals is None:
            ag = torch.empty(2, dtype=torch.float32, device=dev)
        else:
            ag, mode = act_globals, GLOBAL_GIVEN
    L = lib()
    ws = _workspace(L.moe_grouped_nvfp4_ffn_workspace_size(T, H, I, E, k, act), dev, workspace)
    cw = weights.c_struct()
    _check(L.moe_grouped_nvfp4_ffn(_ptr(x), T, H, I, E, k, _ptr(topk_ids), _ptr(topk_weights),
                                   _ptr(expert_offsets), _ptr(sorted_pairs), ctypes.byref(cw),
                                   act, mode, _ptr(ag), _ptr(y), _dt(y.dtype), _ptr(ws),
                                   ws.numel(), _stream()))
    return y, ag


def moe_route_ffn_decode(logits, x, weights: ExpertWeights, k, renormalize=True,
                         out_dtype=torch.bfloat16, route_out=None, out=None, workspace=None):
    """Routing and the routed-expert FFN of a decode batch (W4A16) in two
    launches, bit-identical to moe_route_topk then moe_grouped_nvfp4_ffn.
    Returns (y [T,H], (topk_ids, topk_weights, expert_offsets, sorted_pairs))."""
    T, H = x.shape
    E, I = weights.num_experts, weights.intermediate
    dev = x.device
    if route_out is None:
        route_out = (torch.empty((T, k), dtype=torch.int32, device=dev),
                     torch.empty((T, k), dtype=torch.float32, device=dev),
                     torch.empty(E + 1, dtype=torch.int32, device=dev),
                     torch.empty(T * k, dtype=torch.int32, device=dev))
    ids, w, off, pairs = route_out
    y = out if out is not None else torch.empty((T, H), dtype=out_dtype, device=dev)
    L = lib()
    ws = _workspace(L.moe_route_ffn_decode_workspace_size(T, H, I, E, k), dev, workspace)
    cw = weights.c_struct()
    _check(L.moe_route_ffn_decode(_ptr(logits), _ptr(x), T, H, I, E, k, int(bool(renormalize)),
                                  _ptr(ids), _ptr(w), _ptr(off), _ptr(pairs), ctypes.byref(cw),
                                  _ptr(y), _dt(y.dtype), _ptr(ws), ws.numel(), _stream()))
    return y, route_out


def route_ffn_decode_supported(T, H, I, E, k):
    """Whether moe_route_ffn_decode takes this shape (the fused decode path)."""
    return (H == 2048 and I > 0 and I % 256 == 0 and 1 <= k <= 8 and k <= E <= 512
            and T * k <= 256 and 2 * T * k <= 32 * E)


def moe_grouped_nvfp4_ffn_static(x, weights: ExpertWeights, topk_ids, topk_weights,
                                 expert_offsets, sorted_pairs, k, act=W4A16, act_globals=None,
                                 out_dtype=torch.bfloat16, out=None):
    """moe_grouped_nvfp4_ffn on the library's static scratch (no workspace, no
    allocation inside the call).  Returns (y [T,H], act_globals or None)."""
    T, H = x.shape
    E, I = weights.num_experts, weights.intermediate
    y = out if out is not None else torch.empty((T, H), dtype=out_dtype, device=x.device)
    mode, ag = GLOBAL_COMPUTE, None
    if act == W4A4:
        if act_globals is None:
            ag = torch.empty(2, dtype=torch.float32, device=x.device)
        else:
            ag, mode = act_globals, GLOBAL_GIVEN
    cw = weights.c_struct()
    _check(lib().moe_grouped_nvfp4_ffn_static(
        _ptr(x), T, H, I, E, k, _ptr(topk_ids), _ptr(topk_weights), _ptr(expert_offsets),
        _ptr(sorted_pairs), ctypes.byref(cw), act, mode, _ptr(ag), _ptr(y), _dt(y.dtype),
        _stream()))
    return y, ag


def ffn_debug_h(workspace, T, H, I, E, k, act=W4A16, given=False):
    """The h rows a moe_grouped_nvfp4_ffn call (same arguments, this thread)
    left in `workspace`: (h_bf16 [T*k, I] as float32 or None, h_operand
    [T*k, I] float32 (W4A4 e2m1*e4m3 values) or None), rows in expert-sorted
    position order."""
    ho, hq = _sz(), _sz()
    mask = lib().moe_grouped_nvfp4_ffn_debug_h(T, H, I, E, k, act,
                                               GLOBAL_GIVEN if given else GLOBAL_COMPUTE,
                                               ctypes.byref(ho), ctypes.byref(hq))
    P = T * k
    raw = workspace.view(torch.uint8)
    hb = hqv = None
    if mask & 1:
        hb = raw[ho.value: ho.value + 2 * P * I].view(torch.bfloat16).view(P, I).float()
    if mask & 2:
        hqv = raw[hq.value: hq.value + 2 * P * I].view(torch.float16).view(P, I).float()
    return hb, hqv


def read_probe(buf, sink):
    """A plain streaming read of buf (device memory; a measurement aid)."""
    _check(lib().nvfp4_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                  _stream()))


def set_ffn_separate_h_quant(separate):
    """W4A4 with given globals: quantise h in a pass of its own (True) rather
    than in the gate/up epilogue (False, the default).  Per calling thread;
    the outputs are bit-identical either way."""
    lib().nvfp4_set_ffn_separate_h_quant(1 if separate else 0)
