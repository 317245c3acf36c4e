"""moe_layer_forward_static (no workspace argument: a static device scratch
array) against moe_layer_forward with a caller workspace, through the C ABI:
two calls in a row, the second with a smaller input, each bit-equal; a call
whose workspace exceeds the array is refused."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from block_scaled_fp4_gemv_amd import binding as B  # noqa: E402

from helpers import Layer, iid_tokens  # noqa: E402

pytestmark = pytest.mark.gpu


def _static(fmt, pool, stride, H, F, E, k, x, R):
    T = x.shape[0]
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), -7.0, dtype=torch.float32, device="cuda")
    out = torch.full((T, H), 0x7777, dtype=torch.uint16, device="cuda")
    p = B._ptr
    st = B.lib().moe_layer_forward_static(fmt, p(pool), stride, H, F, E, k, 0, p(x), T, p(R), p(idx), p(w),
                                          p(out), None)
    return st, idx, w, out


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_static_scratch_equals_caller_workspace(fmt):
    H, E, F, k = 2048, 64, 512, 8
    L = Layer(fmt, H, E, F, cfg=51, layer=0, w_std=0.02)
    pool, R = L.device()
    # 96 tokens (grouped prefill path, 4.6 MiB of workspace), then 1 token
    # (decode path) into the same array
    for T in (96, 1):
        x = torch.from_numpy(iid_tokens(0, 51, T, H, [L.router], k)).cuda()
        st, idx, w, out = _static(fmt, pool, L.stride, H, F, E, k, x, R)
        assert st == B.MOE_OK, B.lib().moe_last_error()
        ref = B.moe_layer_forward(fmt, pool, L.stride, H, F, E, k, x, R)
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]) and torch.equal(w, ref[1]) and torch.equal(out, ref[2]), (fmt, T)


def test_static_scratch_refuses_a_larger_workspace():
    fmt, H, E, F, k, T = 1, 2048, 256, 512, 8, 2048
    assert B.moe_layer_workspace(fmt, T, H, F, k, E) > (32 << 20)
    x = torch.zeros((T, H), dtype=torch.uint16, device="cuda")
    R = torch.zeros((E, H), dtype=torch.float32, device="cuda")
    pool = torch.zeros(E * B.blob_stride(fmt, H, F), dtype=torch.uint8, device="cuda")
    st, idx, w, out = _static(fmt, pool, B.blob_stride(fmt, H, F), H, F, E, k, x, R)
    torch.cuda.synchronize()
    assert st == B.MOE_E_WORKSPACE
    assert bool((out == 0x7777).all()) and bool((idx == -7).all())
