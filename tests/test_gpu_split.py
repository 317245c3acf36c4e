"""GPU parity of the cached layer with a share q of each step's misses computed
on the host CPU (moe_cached_layer_forward_split): the LRU follows the oracle
exactly whatever q is; the output equals the all-resident layer bit for bit on
steps where no pair is CPU-served, and meets the oracle layer at the output
tolerance on every step; the CPU-served experts still land in their slots."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from block_scaled_fp4_gemv_amd import binding as B  # noqa: E402
from oracle import formats as fm, lru as olru, moe  # noqa: E402

from helpers import Layer, ar1_states, assert_rows_close, bf16_dev_to_f64  # noqa: E402

pytestmark = pytest.mark.gpu
NV, MX = 1, 2


@pytest.mark.parametrize("fmt,H,E,F,k,S,q,n_steps", [(NV, 256, 16, 512, 2, 6, 0.0, 12), (NV, 256, 16, 512, 2, 6, 0.5, 20),
                                                      (MX, 256, 16, 512, 2, 6, 1.0, 16),
                                                      (NV, 2048, 256, 512, 8, 64, 0.5, 16)])
def test_cached_layer_split(fmt, H, E, F, k, S, q, n_steps):
    L = Layer(fmt, H, E, F, cfg=91, layer=0, w_std=0.02)
    xs = ar1_states(0, 91, n_steps, H, [L.router], k)
    hp = L.host_pool()
    pool_res, R = torch.from_numpy(hp).cuda(), torch.from_numpy(np.ascontiguousarray(L.router)).cuda()
    host = torch.empty(E * L.stride, dtype=torch.uint8).pin_memory()
    host.numpy()[:] = hp
    slots = torch.zeros(S * L.stride, dtype=torch.uint8, device="cuda")
    cl = B.CachedLayer(R, host, slots, E, S, 1, k)
    ws = torch.empty(B.moe_cached_layer_workspace(fmt, 1, H, F, k, E) + 256, dtype=torch.uint8, device="cuda")
    hws = B.new_split_host_workspace(1, H, F, k)
    defer = torch.cuda.Event()
    copy = torch.cuda.Stream()
    ref = olru.StampLRU(E, S)
    eb = B.moe_expert_bytes(fmt, H, F)
    bufs = [torch.empty(s_, dtype=d, device="cuda") for s_, d in
            (((1, k), torch.int32), ((1, k), torch.float32), (k, torch.int32), (k, torch.int32), ((1, H), torch.uint16))]
    idx, w, pair_slot, pair_order, out = bufs
    total_cpu = 0
    for t in range(n_steps):
        xd = torch.from_numpy(np.ascontiguousarray(xs[t:t + 1])).cuda()
        hits, miss, n_cpu = B.moe_cached_layer_forward_split(fmt, L.stride, H, F, E, k, cl, xd, idx, w, pair_slot,
                                                             pair_order, out, ws, q, hws, defer, copy_stream=copy)
        torch.cuda.current_stream().wait_event(defer)
        torch.cuda.synchronize()
        tag = f"step {t}"
        r = ref.step(idx.cpu().numpy().ravel())
        assert (hits, miss) == (r["n_hits"], r["n_miss"]) and n_cpu == int(q * miss), tag
        assert np.array_equal(cl.lru.slot_expert.cpu().numpy(), ref.slot_expert), tag
        assert np.array_equal(pair_slot.cpu().numpy(), r["pair_slot"]), tag
        o = moe.moe_layer(fmt, xs[t:t + 1], L.router, L.experts, k)
        assert np.array_equal(idx.cpu().numpy(), o["idx"]), tag
        assert_rows_close(bf16_dev_to_f64(out), fm.bf16_to_f64(o["out"]), what=f"out {tag}")
        if n_cpu == 0:
            _, _, out_r = B.moe_layer_forward(fmt, pool_res, L.stride, H, F, E, k, xd, R)
            torch.cuda.synchronize()
            assert torch.equal(out, out_r), tag
        total_cpu += n_cpu
        for s_, e_ in enumerate(ref.slot_expert):
            if e_ >= 0:
                assert np.array_equal(slots[s_ * L.stride:s_ * L.stride + eb].cpu().numpy(),
                                      hp[e_ * L.stride:e_ * L.stride + eb]), f"{tag} slot {s_}"
    assert (total_cpu > 0) == (q > 0)
