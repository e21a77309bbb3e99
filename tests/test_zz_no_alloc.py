"""The FFN entry point without a workspace (moe_grouped_nvfp4_ffn_static,
for callers that cannot allocate): its output equals the workspace entry
point's bit for bit, on two calls in a row through the one static scratch
array of the device, the second with a smaller input (so stale contents of
the first call are present), in W4A16 and W4A4 with online globals.  Every
call goes through the C ABI."""
import sys

import numpy as np
import pytest
import torch

from nvfp4_routed_expert_amd import native, synth, weights

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _inputs(T, H, I, E, k, seed, zipf=None):
    x = synth.activations(T, H, seed).to(DEV)
    logits = torch.from_numpy(synth.router_logits(T, E, seed, zipf_s=zipf)).to(DEV)
    w = weights.synthetic_experts(E, H, I, seed, DEV)
    ids, wts, off, pairs = native.moe_route_topk(logits, k)
    return x, w, ids, wts, off, pairs


@pytest.mark.parametrize("act", [native.W4A16, native.W4A4])
def test_static_scratch_ffn_equals_workspace_ffn(act):
    L = native.lib()
    cases = [(512, 2048, 512, 512, 8, 1.1),   # the 512-token chunk: tile path, large scratch
             (16, 2048, 512, 512, 8, None),   # then decode: a smaller call on the same array
             (8, 1024, 768, 1, 1, None),      # a dense MLP of 8 rows (bf16 GEMV, split K)
             (1, 1024, 2048, 1, 1, None)]     # and of one row (the one-row kernels)
    if act == native.W4A4:
        cases = [(512, 1024, 512, 64, 4, None), (24, 512, 256, 16, 2, None)]
    for T, H, I, E, k, zipf in cases:
        say("static scratch ffn", T, H, I, E, k, act)
        need = L.moe_grouped_nvfp4_ffn_workspace_size(T, H, I, E, k, act)
        assert 0 < need <= L.moe_grouped_nvfp4_ffn_static_max_bytes()
        x, w, ids, wts, off, pairs = _inputs(T, H, I, E, k, 3, zipf)
        for dt in (torch.float32, torch.bfloat16):
            y_ws, g_ws = native.moe_grouped_nvfp4_ffn(x, w, ids, wts, off, pairs, k, act=act,
                                                      out_dtype=dt)
            y_st, g_st = native.moe_grouped_nvfp4_ffn_static(x, w, ids, wts, off, pairs, k,
                                                             act=act, out_dtype=dt)
            torch.cuda.synchronize()
            assert torch.equal(y_st, y_ws), (T, H, I, E, k, dt)
            if act == native.W4A4:
                assert torch.equal(g_st, g_ws)


def test_static_scratch_rejects_shapes_beyond_its_size():
    """A batch whose scratch exceeds the static array is refused before
    anything is enqueued, with a message that names both sizes."""
    L = native.lib()
    T, H, I, E, k = 2048, 4096, 1536, 128, 8
    need = L.moe_grouped_nvfp4_ffn_workspace_size(T, H, I, E, k, native.W4A4)
    assert need > L.moe_grouped_nvfp4_ffn_static_max_bytes()
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    w = weights.empty_experts(E, H, I, DEV)
    i32 = dict(dtype=torch.int32, device=DEV)
    ids, off, pairs = torch.zeros((T, k), **i32), torch.zeros(E + 1, **i32), torch.zeros(T * k, **i32)
    wts = torch.zeros((T, k), dtype=torch.float32, device=DEV)
    with pytest.raises(native.NVFP4Error) as ei:
        native.moe_grouped_nvfp4_ffn_static(x, w, ids, wts, off, pairs, k, act=native.W4A4)
    assert ei.value.status == 4 and str(need) in str(ei.value)
