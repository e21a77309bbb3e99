"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/nvfp4moe.h declares, and rejects bad arguments with
the documented status before enqueuing anything."""
import ctypes
import os
import re

import pytest

from nvfp4_routed_expert_amd import native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(native.LIB_PATH),
                                reason="library not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for call in ("nvfp4_quantize", "nvfp4_linear", "moe_route_topk", "moe_grouped_nvfp4_ffn",
                 "moe_router_topk", "moe_shared_expert_ffn"):
        assert call in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(native.LIB_PATH)
    names = declared_functions()
    assert names and sorted(names) == sorted(native.exported_symbols())
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = native.lib()
    for code, text in [(0, b"ok"), (1, b"invalid argument"), (2, b"unsupported shape"),
                       (3, b"misaligned pointer"), (4, b"workspace too small"),
                       (5, b"HIP error")]:
        assert L.nvfp4_status_string(code) == text
    assert L.nvfp4_status_string(99) == b"unknown status"


FAKE = ctypes.c_void_p(1 << 20)          # aligned, never dereferenced
FAKE_MIS = ctypes.c_void_p((1 << 20) + 4)


def _last():
    return native.lib().nvfp4_last_error().decode()


def test_quantize_validation():
    L = native.lib()
    ws = L.nvfp4_quantize_workspace_size(4, 64)
    assert ws > 0
    q = lambda x, rows, cols, ld, codes, wsb, mode=0: L.nvfp4_quantize(
        x, 0, rows, cols, ld, codes, FAKE, FAKE, mode, FAKE, wsb, None)
    assert q(None, 4, 64, 64, FAKE, ws) == 1 and "x is NULL" in _last()
    assert q(FAKE, 4, 48, 48, FAKE, ws) == 2 and "multiple of 32" in _last()
    assert q(FAKE, 0, 64, 64, FAKE, ws) == 1
    assert q(FAKE, 4, 64, 32, FAKE, ws) == 1 and "ld_x" in _last()
    assert q(FAKE, 4, 64, 64, FAKE_MIS, ws) == 3 and "codes" in _last()
    assert q(FAKE, 4, 64, 64, FAKE, ws - 1) == 4
    assert q(FAKE, 4, 64, 64, FAKE, ws, mode=7) == 1


def test_linear_validation():
    L = native.lib()
    m = native.Matrix(FAKE.value, FAKE.value, FAKE.value, 64, 96)   # K = 96 fine
    ws = L.nvfp4_linear_workspace_size(4, 64, 96, 0)
    lin = lambda M, mat, act=0, y=FAKE, wsb=ws: L.nvfp4_linear(
        FAKE, M, ctypes.byref(mat), act, 0, None, y, 0, FAKE, wsb, None)
    assert lin(-1, m) == 1
    assert L.nvfp4_linear(None, 0, ctypes.byref(m), 0, 0, None, None, 0, None, 0, None) == 0
    assert lin(0, bad := native.Matrix(FAKE.value, FAKE.value, FAKE.value, 64, 80)) == 2
    bad = native.Matrix(FAKE.value, FAKE.value, FAKE.value, 64, 80)
    assert lin(4, bad) == 2
    assert lin(4, m, act=3) == 1
    assert lin(4, m, y=None) == 1
    assert lin(4, m, y=FAKE_MIS) == 3
    assert lin(4, m, wsb=ws - 256) == 4
    nullm = native.Matrix(None, FAKE.value, FAKE.value, 64, 96)
    assert lin(4, nullm) == 1 and "codes" in _last()
    # W4A4 with a given scale needs the pointer
    assert L.nvfp4_linear(FAKE, 4, ctypes.byref(m), 1, 1, None, FAKE, 0, FAKE, ws, None) == 1


def test_route_validation():
    L = native.lib()
    r = lambda T, E, k, logits=FAKE: L.moe_route_topk(logits, T, E, k, 1, FAKE, FAKE, FAKE,
                                                      FAKE, None, 0, None)
    assert r(16, 512, 0) == 2
    assert r(16, 8, 9) == 2
    assert r(16, 2048, 8) == 2
    assert r(16, 64, 33) == 2
    assert r(-1, 64, 8) == 1
    assert r(0, 2048, 8) == 2          # an empty batch still checks E and k
    assert r(16, 64, 8, logits=None) == 1
    assert r(16, 64, 8, logits=FAKE_MIS) == 3
    assert r((1 << 22), 64, 8) == 2
    assert r(16, 64, 8) == 4 and "workspace" in _last()
    # the top-k alone: both permutation outputs NULL (no workspace needed);
    # one of them NULL is a missing argument
    assert L.moe_route_topk(FAKE, 16, 64, 8, 1, FAKE, FAKE, None, FAKE, FAKE, 256, None) == 1
    assert L.moe_route_topk(FAKE, 16, 64, 8, 1, FAKE, FAKE, FAKE, None, FAKE, 256, None) == 1
    assert L.moe_route_topk(FAKE_MIS, 16, 64, 8, 1, FAKE, FAKE, None, None, None, 0, None) == 3


def test_route_ffn_decode_validation():
    """moe_route_ffn_decode takes only the fused decode shapes and checks its
    arguments before anything is enqueued."""
    L = native.lib()
    w = native.ExpertWeightsC(*([FAKE.value] * 9))
    T, H, I, E, k = 16, 2048, 512, 512, 8
    ws = L.moe_route_ffn_decode_workspace_size(T, H, I, E, k)
    assert ws >= T * k * (I // 256) * H * 4
    f = lambda T=T, H=H, I=I, E=E, k=k, wsb=ws, lg=FAKE, off=FAKE, dt=0: L.moe_route_ffn_decode(
        lg, FAKE, T, H, I, E, k, 1, FAKE, FAKE, off, FAKE, ctypes.byref(w), FAKE, dt, FAKE, wsb,
        None)
    assert f(H=4096) == 2 and "fused decode path" in _last()
    assert f(I=384) == 2
    assert f(k=9) == 2
    assert f(E=600) == 2
    assert f(T=64) == 2                  # T*k > 256
    assert f(T=32, E=4, k=4) == 2        # 2*T*k > 32*E
    assert f(T=-1) == 1
    assert f(lg=None) == 1 and "logits" in _last()
    assert f(off=None) == 1
    assert f(dt=7) == 1
    assert f(wsb=ws - 1) == 4
    assert f(lg=FAKE_MIS) == 3


def test_ffn_validation():
    L = native.lib()
    w = native.ExpertWeightsC(*([FAKE.value] * 9))
    T, H, I, E, k = 16, 256, 128, 8, 2
    ws = L.moe_grouped_nvfp4_ffn_workspace_size(T, H, I, E, k, 0)
    assert ws > 0
    f = lambda T=T, H=H, I=I, E=E, k=k, wsb=ws, ww=w, act=0, ids=FAKE: L.moe_grouped_nvfp4_ffn(
        FAKE, T, H, I, E, k, ids, FAKE, FAKE, FAKE, ctypes.byref(ww), act, 0, None, FAKE, 0,
        FAKE, wsb, None)
    assert f(H=250) == 2
    assert f(I=100) == 2
    assert f(k=9) == 2
    assert f(T=-1) == 1
    # an empty batch: no launch, its arrays may be NULL, weights still checked
    assert L.moe_grouped_nvfp4_ffn(None, 0, H, I, E, k, None, None, None, None, ctypes.byref(w),
                                   0, 0, None, None, 0, None, 0, None) == 0
    assert f(T=0, H=250) == 2
    assert f(wsb=ws - 1) == 4
    assert f(act=5) == 1
    assert f(ids=None) == 1 and "topk_ids" in _last()
    assert f(ids=FAKE_MIS) == 3
    bad = native.ExpertWeightsC(*([FAKE.value] * 8 + [None]))
    assert f(ww=bad) == 1 and "down_global" in _last()
    mis = native.ExpertWeightsC(*([FAKE_MIS.value] + [FAKE.value] * 8))
    assert f(ww=mis) == 3
    # a W4A4 call with given globals needs them
    assert L.moe_grouped_nvfp4_ffn(FAKE, T, H, I, E, k, FAKE, FAKE, FAKE, FAKE, ctypes.byref(w), 1,
                                   1, None, FAKE, 0, FAKE, ws, None) == 1
    # no permutation (both NULL) only on the fused decode path; one NULL alone
    # is a missing argument everywhere
    g = lambda off, pairs, H=H, I=I, E=E, k=k, act=0: L.moe_grouped_nvfp4_ffn(
        FAKE, T, H, I, E, k, FAKE, FAKE, off, pairs, ctypes.byref(w), act, 0, None, FAKE, 0, FAKE,
        L.moe_grouped_nvfp4_ffn_workspace_size(T, H, I, E, k, act), None)
    assert g(None, None) == 1 and "fused decode path" in _last()      # H = 256
    assert g(None, None, H=2048, I=512, E=512, k=8, act=1) == 1      # W4A4
    assert g(None, FAKE, H=2048, I=512, E=512, k=8) == 1
    assert g(FAKE, None, H=2048, I=512, E=512, k=8) == 1


def test_router_validation():
    L = native.lib()
    T, H, E, k = 16, 256, 64, 8
    ws = L.moe_router_topk_workspace_size(T, H, E, k)
    assert ws > 0
    r = lambda T=T, H=H, E=E, k=k, x=FAKE, rw=FAKE, bias=None, lg=None, ids=FAKE, wsb=ws: \
        L.moe_router_topk(x, T, H, rw, bias, E, k, 1, lg, ids, FAKE, FAKE, FAKE, FAKE, wsb, None)
    assert r(H=100) == 2 and "H" in _last()
    assert r(E=0) == 2
    assert r(E=2048) == 2
    assert r(k=0) == 2
    assert r(k=65) == 2
    assert r(T=-1) == 1
    assert r(x=None) == 1 and "x" in _last()
    assert r(rw=None) == 1 and "router_w" in _last()
    assert r(ids=None) == 1
    assert r(x=FAKE_MIS) == 3
    assert r(rw=FAKE_MIS) == 3
    assert r(bias=FAKE_MIS) == 3 and "router_bias" in _last()
    assert r(lg=FAKE_MIS) == 3 and "logits" in _last()
    assert r(wsb=ws - 1) == 4
    # the workspace grows with the partial sums of the K split
    assert L.moe_router_topk_workspace_size(16, 2048, 512, 8) > ws


def test_shared_expert_validation():
    L = native.lib()
    T, H, I = 16, 256, 128
    ws = L.moe_shared_expert_ffn_workspace_size(T, H, I)
    assert ws > 0
    f = lambda T=T, H=H, I=I, x=FAKE, wg=FAKE, wu=FAKE, wd=FAKE, y=FAKE, dt=0, wsb=ws: \
        L.moe_shared_expert_ffn(x, T, H, I, wg, wu, wd, 0, y, dt, FAKE, wsb, None)
    assert f(H=100) == 2
    assert f(I=48) == 2
    assert f(T=-1) == 1
    assert f(T=0, x=None, y=None, wsb=0) == 0        # an empty batch: no launch
    assert f(T=0, x=None, y=None, wg=None) == 1
    assert f(wg=None) == 1 and "w_gate" in _last()
    assert f(wd=None) == 1 and "w_down" in _last()
    assert f(y=None) == 1
    assert f(dt=7) == 1 and "y_dtype" in _last()
    assert f(wu=FAKE_MIS) == 3
    assert f(y=FAKE_MIS) == 3
    assert f(wsb=ws - 1) == 4
    assert L.moe_shared_expert_ffn_workspace_size(0, H, I) == 0


def test_expert_cache_validation():
    L = native.lib()
    assert L.moe_expert_cache_init(FAKE, 0, FAKE, FAKE, FAKE, 8, None) == 2
    assert L.moe_expert_cache_init(FAKE, 64, FAKE, FAKE, FAKE, 2048, None) == 2
    assert L.moe_expert_cache_init(None, 64, FAKE, FAKE, FAKE, 8, None) == 1
    plan = lambda T=4, k=2, E=64, S=16, step=1, prot=1, ids=FAKE, mx=8: L.moe_expert_cache_plan(
        ids, T, k, E, S, FAKE, FAKE, FAKE, FAKE, step, prot, mx, FAKE, FAKE, FAKE, None)
    assert plan(E=2000) == 2
    assert plan(S=0) == 2
    assert plan(T=-1) == 1
    assert plan(step=0, prot=0) == 1
    assert plan(step=3, prot=4) == 1
    assert plan(ids=None) == 1
    assert plan(mx=-1) == 1 and "max_fetch" in _last()
    assert plan(mx=1025) == 1
    w = native.ExpertWeightsC(*([FAKE.value] * 9))
    mis = native.ExpertWeightsC(*([FAKE_MIS.value] + [FAKE.value] * 8))
    odd_g = native.ExpertWeightsC(*([FAKE.value] * 8 + [FAKE.value + 2]))
    nul = native.ExpertWeightsC(*([FAKE.value] * 8 + [None]))
    f = lambda hw=w, pw=w, H=256, I=128, mx=8: L.moe_expert_cache_fetch(
        ctypes.byref(hw), ctypes.byref(pw), H, I, FAKE, FAKE, mx, None)
    assert f(H=100) == 2
    assert f(mx=-1) == 1
    assert f(hw=nul) == 1 and "host_w" in _last()
    assert f(pw=mis) == 3 and "pool" in _last()
    assert f(pw=odd_g) == 3
    pp = lambda T=4, E=64, k=2, ids=FAKE: L.moe_permute_pairs(ids, T, E, k, FAKE, FAKE, None)
    assert pp(E=0) == 2
    assert pp(k=33) == 2
    assert pp(T=-1) == 1
    assert pp(ids=FAKE_MIS) == 3


def test_route_workspace_init_validation():
    """moe_route_workspace_init checks its workspace on the host before any
    launch (NULL, misaligned, fewer than 4 bytes), and the binding's routing
    workspaces go through it (no caller relies on a zeroed allocation)."""
    L = native.lib()
    assert L.moe_route_workspace_init(None, 256, None) == 1
    assert L.moe_route_workspace_init(FAKE_MIS, 256, None) == 3
    assert L.moe_route_workspace_init(FAKE, 3, None) == 4
    import inspect
    assert "_init_route_workspace" in inspect.getsource(native.route_workspace)
    assert "_init_route_workspace" in inspect.getsource(native.router_workspace)


def test_ffn_debug_h_layout():
    """The debug query places h and its W4A4 operand where the FFN's
    workspace holds them, inside the workspace, and names what each path
    leaves there."""
    L = native.lib()
    ho, hq = ctypes.c_size_t(), ctypes.c_size_t()
    for T, H, I, E, k, act, given, want in [
            (2048, 4096, 1536, 128, 8, 1, 0, 3),    # W4A4 online: bf16 h, then its operand
            (2048, 4096, 1536, 128, 8, 1, 1, 2),    # W4A4 given: h quantised in the epilogue
            (512, 2048, 512, 512, 8, 0, 0, 1),      # W4A16 tiles: bf16 h
            (16, 2048, 512, 512, 8, 0, 0, 0),       # decode rows: h stays in LDS
            (16, 2048, 512, 512, 8, 1, 0, 3)]:      # W4A4 decode GEMV
        m = L.moe_grouped_nvfp4_ffn_debug_h(T, H, I, E, k, act, given, ctypes.byref(ho),
                                            ctypes.byref(hq))
        assert m == want, (T, H, I, E, k, act, given, m)
        ws = L.moe_grouped_nvfp4_ffn_workspace_size(T, H, I, E, k, act)
        P = T * k
        assert ho.value >= 2 * T * H and hq.value >= ho.value + 2 * P * I
        assert hq.value + 2 * P * I <= ws


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(native, "_LIB", None)
    monkeypatch.setattr(native, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        native.lib()


def test_ffn_workspace_holds_the_fused_decode_partials():
    """The fused decode FFN keeps a partial output row per pair and
    256-column slice of I (fp32): the workspace query covers them."""
    L = native.lib()
    for T, H, I, E, k in [(16, 2048, 512, 512, 8), (16, 2048, 1024, 64, 8), (4, 2048, 768, 16, 3)]:
        need = T * k * (I // 256) * H * 4
        assert L.moe_grouped_nvfp4_ffn_workspace_size(T, H, I, E, k, 0) >= need


def test_bench_names_the_kernel_the_library_dispatches():
    """The bench's roofline line names the gate/up kernel by mirroring the
    library's dispatch: decode-sized batches stream rows (both projections
    in one kernel at H = 2048), larger ones tile."""
    import bench
    assert bench.gate_up_kernel(16, 2048, 512, 512, 8, "w4a16") == "row_ffn_kernel"
    assert bench.gate_up_kernel(16, 2048, 2080, 512, 8, "w4a16") == "row_gemv_kernel"
    assert bench.gate_up_kernel(16, 1024, 512, 512, 8, "w4a16") == "row_gemv_kernel"
    assert bench.gate_up_kernel(512, 2048, 512, 512, 8, "w4a16") == "tile_gemm_kernel"
    assert bench.gate_up_kernel(2048, 4096, 1536, 128, 8, "w4a4") == "tile_gemm_kernel"
    assert bench.gate_up_kernel(1, 5120, 17408, 1, 1, "w4a16") == "row_mlp_gate_up_kernel"
    assert bench.gate_up_kernel(1, 6144, 17408, 1, 1, "w4a16") == "row_gemv_kernel"
    assert bench.gate_up_kernel(2, 5120, 17408, 1, 1, "w4a16") == "row_gemv_kernel"
    assert bench.gate_up_kernel(8, 5120, 17408, 1, 1, "w4a16") == "dense_gemv_kernel"
    assert bench.gate_up_kernel(32, 5120, 17408, 1, 1, "w4a16") == "dense_gemv_kernel"
    assert bench.gate_up_kernel(33, 5120, 17408, 1, 1, "w4a16") == "tile_gemm_kernel"
    assert bench.gate_up_kernel(16, 2048, 512, 512, 8, "w4a4") == "grouped_gemv_kernel"
    assert bench.gate_up_kernel(300, 96, 64, 4, 2, "w4a16") == "grouped_gemm_kernel"


def test_bench_and_entry_reference_only_defined_names():
    """Every name bench.py and __graft_entry__.py load at module or function
    level is bound somewhere in the file, imported, or a builtin: a helper
    dropped in an edit (a flag whose handler no longer exists) fails here
    rather than on the GPU machine."""
    import ast
    import builtins
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for fname in ("bench.py", "__graft_entry__.py"):
        tree = ast.parse(open(os.path.join(root, fname)).read())
        bound = set(dir(builtins)) | {"__file__"}
        for node in ast.walk(tree):
            if isinstance(node, (ast.FunctionDef, ast.ClassDef)):
                bound.add(node.name)
            elif isinstance(node, (ast.Import, ast.ImportFrom)):
                bound |= {(a.asname or a.name).split(".")[0] for a in node.names}
            elif isinstance(node, ast.arg):
                bound.add(node.arg)
            elif isinstance(node, ast.ExceptHandler) and node.name:
                bound.add(node.name)
            elif isinstance(node, ast.Name) and isinstance(node.ctx, ast.Store):
                bound.add(node.id)
        used = {n.id for n in ast.walk(tree) if isinstance(n, ast.Name) and isinstance(n.ctx, ast.Load)}
        assert not (used - bound), (fname, sorted(used - bound))

