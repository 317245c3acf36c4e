"""Prepared routers (moe_router_prepare, MOE_ROUTE_PREPARED): the fp32 router
followed by its exact three-term bf16 split, built once per weight set.

Routing and whole layers through a prepared router must equal those through
the plain fp32 router bit for bit (the plain path is pinned to the oracle by
the routing tests), at token counts that take the router GEMV (T <= 4), the
router GEMM and the permutation's one-batch and multi-batch paths.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from block_scaled_fp4_gemv_amd import binding as B  # noqa: E402
from block_scaled_fp4_gemv_amd import synth as sy  # noqa: E402
from oracle import formats as fm  # noqa: E402

from helpers import Layer, iid_tokens  # noqa: E402

pytestmark = pytest.mark.gpu
NV = 1


def _x_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def test_prepared_router_layout():
    """The fp32 part is the router; hi + mid + lo of the planes equals every
    router weight exactly, for magnitudes from 1e-30 to 1e30, the ends of the
    exact range (2^-100, 3e38) and signed zeros."""
    E, H = 64, 256
    rng = np.random.default_rng(3)
    R = (rng.normal(0, 1, (E, H)) * 10.0 ** rng.integers(-30, 31, (E, H))).astype(np.float32)
    R[0, :8] = [0.0, -0.0, 1.0, -1.0, 2.0 ** -100, -(2.0 ** -100) * 1.2345, 3.0e38, -3.0e38]
    P = B.PreparedRouter(torch.from_numpy(R).cuda())
    torch.cuda.synchronize()
    buf = P.buf.cpu().numpy()
    n = E * H
    assert np.array_equal(buf[:4 * n].view(np.float32).reshape(E, H), R)
    off = (4 * n + 255) // 256 * 256
    planes = buf[off:off + 6 * n].view(np.uint16).reshape(3, E, H)
    total = sum(fm.bf16_to_f64(planes[p]) for p in range(3))
    assert np.array_equal(total, R.astype(np.float64))


@pytest.mark.parametrize("E", [64, 256])
@pytest.mark.parametrize("T", [1, 4, 5, 300, 2100])
def test_prepared_route_equals_plain(E, T):
    H, k = 2048, 8
    R = sy.router(0, 21, 0, E, H)
    x = _x_dev(iid_tokens(0, 21, T, H, [R], k))
    Rd = torch.from_numpy(R).cuda()
    P = B.PreparedRouter(Rd)
    for flags in (0, B.MOE_ROUTE_RENORM):
        a = B.moe_route(x, Rd, k, flags=flags)
        b = B.moe_route(x, P, k, flags=flags)
        torch.cuda.synchronize()
        for u, v, what in zip(a, b, ("topk_idx", "topk_w", "pair_perm", "expert_off")):
            assert torch.equal(u, v), (what, flags)


@pytest.mark.parametrize("T", [1, 3, 2048])
def test_prepared_layer_equals_plain(T):
    """The 35B-shape layer (NVFP4, 256 experts, top-8) through a prepared router:
    decode (T <= 4: router GEMV + in-block top-k) and 2048-token prefill."""
    H, E, F, k = 2048, 256, 512, 8
    L = Layer(NV, H, E, F, cfg=22, layer=0, w_std=0.02)
    pool, Rd = L.device()
    x = _x_dev(iid_tokens(0, 22, T, H, [L.router], k))
    P = B.PreparedRouter(Rd)
    a = B.moe_layer_forward(NV, pool, L.stride, H, F, E, k, x, Rd)
    b = B.moe_layer_forward(NV, pool, L.stride, H, F, E, k, x, P)
    torch.cuda.synchronize()
    for u, v, what in zip(a, b, ("topk_idx", "topk_w", "out")):
        assert torch.equal(u, v), what


def test_unknown_route_flags_rejected():
    H, E, k = 256, 16, 2
    R = torch.from_numpy(sy.router(0, 23, 0, E, H)).cuda()
    x = torch.zeros((8, H), dtype=torch.uint16, device="cuda")
    with pytest.raises(B.MoeError):
        B.moe_route(x, R, k, flags=0x400)
