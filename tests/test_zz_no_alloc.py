"""The allocation-free forward (nf4moe_moe_forward_noalloc) against the
forward with a caller workspace (nf4moe_moe_forward), through the C ABI: the
same kernels, so outputs, expert ids and routing weights must agree bit for
bit. Two calls in a row on the library's per-device scratch, the second with
fewer tokens (the scratch keeps the first call's contents), on both kernel
families; and a call too large for the scratch is refused before any work."""
import ctypes

import numpy as np
import pytest

import moe_synth as S
from gpu_helpers import bits_to_torch_bf16, build_layers

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_quantized_moe_expert_amd as M  # noqa: E402

DEV = "cuda"


def _with_workspace(layer, x):
    T = x.shape[0]
    ids = torch.empty(T, layer.top_k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, layer.top_k, dtype=torch.float32, device=DEV)
    out = M.Forward(layer, T, DEV)(x, topk_ids=ids, topk_w=w)
    return out, ids, w


def _noalloc(layer, x):
    """Straight through the C ABI."""
    T = x.shape[0]
    out = torch.full((T, layer.H), float("nan"), dtype=torch.bfloat16, device=DEV)
    ids = torch.full((T, layer.top_k), -1, dtype=torch.int32, device=DEV)
    w = torch.full((T, layer.top_k), float("nan"), dtype=torch.float32, device=DEV)
    st = layer.struct()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = M.lib().nf4moe_moe_forward_noalloc(ctypes.byref(st), ctypes.c_void_p(x.data_ptr()), T,
                                            ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ids.data_ptr()),
                                            ctypes.c_void_p(w.data_ptr()), stream)
    M._check(rc)
    return out, ids, w


def _same(a, b, what):
    torch.cuda.synchronize()
    for name, u, v in zip(("out", "topk_ids", "topk_w"), a, b):
        assert torch.equal(u.view(torch.int16 if u.dtype == torch.bfloat16 else torch.int32),
                           v.view(torch.int16 if v.dtype == torch.bfloat16 else torch.int32)), f"{what}: {name}"


@pytest.mark.parametrize("wl,Ts", [
    (S.custom(E=64, top_k=8, H=2048, I=1024, wid=95), (40, 3)),     # MFMA path, then small-M
    (S.custom(E=64, top_k=8, H=2048, I=1024, wid=95), (1, 1)),      # the fused one-token routing twice
    (S.custom(E=16, top_k=4, H=512, I=256, zipf_s=1.2, wid=96), (333, 17)),
])
def test_noalloc_matches_workspace_forward(wl, Ts):
    layer, _, _ = build_layers(wl, 0, DEV, on_device_rng=True)
    X = S.make_x(wl, max(Ts))
    for T in Ts:
        x = bits_to_torch_bf16(X[:T])
        print(f"[no-alloc] {wl.name} T={T}", flush=True)
        _same(_noalloc(layer, x), _with_workspace(layer, x), f"{wl.name} T={T}")
    # the binding's wrapper takes the same route
    x = bits_to_torch_bf16(X[:Ts[-1]])
    out = torch.empty(Ts[-1], wl.H, dtype=torch.bfloat16, device=DEV)
    M.moe_forward_noalloc(layer, x, out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), _with_workspace(layer, x)[0].view(torch.int16))


def test_noalloc_refuses_calls_beyond_its_scratch():
    wl = S.custom(E=64, top_k=8, H=2048, I=1024, wid=95)
    layer, _, _ = build_layers(wl, 0, DEV, on_device_rng=True)
    T = 4096
    assert layer.workspace_bytes(T) > M.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(T, wl.H, dtype=torch.bfloat16, device=DEV)
    out = torch.full((T, wl.H), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(M.Nf4MoeError, match="WORKSPACE"):
        M.moe_forward_noalloc(layer, x, out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)                     # nothing was enqueued
