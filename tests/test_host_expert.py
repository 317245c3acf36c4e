"""The host (CPU) expert FFN of the miss split (moe_host_expert_ffn) against the
oracle: product code computing from packed blobs, checked per pair at the
output tolerance (rel-L2 <= 5e-3, max-abs <= 2e-2 per row).  Runs on the CPU."""
import numpy as np
import pytest

from block_scaled_fp4_gemv_amd import binding as B
from oracle import formats as fm, moe

from helpers import Layer, assert_rows_close, iid_tokens

NV, MX, F8 = 1, 2, 3


@pytest.mark.parametrize("fmt", [NV, MX, F8])
@pytest.mark.parametrize("H,E,F", [(256, 8, 512), (2048, 4, 512)])
def test_host_expert_ffn_matches_the_oracle(fmt, H, E, F):
    L = Layer(fmt, H, E, F, cfg=81, layer=0, w_std=0.02)
    x = iid_tokens(0, 81, 3, H, [L.router], 2)
    pairs = [(t, e) for t in range(3) for e in range(E)][:8]
    blobs = [L.blob(e) for _, e in pairs]
    ys = B.moe_host_expert_ffn(fmt, H, F, blobs, [x[t] for t, _ in pairs], threads=4)
    ref = []
    for t, e in pairs:
        G, U, D = moe.dequant_expert(fmt, L.expert(e))
        _, y = moe.expert_ffn(G, U, D, fm.bf16_to_f64(x[t:t + 1]))
        ref.append(y[0])
    assert_rows_close(ys, np.array(ref), what="host y")


def test_host_expert_ffn_argument_errors():
    L = Layer(NV, 256, 2, 512, cfg=81, layer=0, w_std=0.02)
    blob = L.blob(0)
    x = np.zeros(256, np.uint16)
    assert B.moe_host_expert_ffn(NV, 256, 512, [], []).shape == (0, 256)
    with pytest.raises(B.MoeError):
        B.moe_host_expert_ffn(9, 256, 512, [blob], [x])
    with pytest.raises(B.MoeError):
        B.moe_host_expert_ffn(NV, 100, 512, [blob], [x])
