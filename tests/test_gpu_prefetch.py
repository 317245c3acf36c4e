"""GPU parity of the cached decode layer with predictive prefetch
(moe_cached_layer_enqueue_prefetch): every step's routing and output equal the
all-resident layer bit for bit; the routed lookup's record and the prefetch
step's record (runner-ups ranks k..k+m-1) equal the oracle's two steps
(oracle.lru: StampLRU.step on the routed experts, then prefetch_step on the
ranked top-(k+m)); the state equals the oracle's after both; occupied slots
hold their experts' host blobs once the prefetch stream has been joined.
Inputs keep the top-(k+m+1) logit gaps >= 1e-3, so the oracle's runner-ups are
unambiguous."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from block_scaled_fp4_gemv_amd import binding as B  # noqa: E402
from oracle import formats as fm, lru as olru, moe  # noqa: E402

from helpers import Layer, ar1_states, assert_rows_close, bf16_dev_to_f64  # noqa: E402

pytestmark = pytest.mark.gpu
NV, F8 = 1, 3


def _x_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


@pytest.mark.parametrize("fmt,H,E,F,k,S,m,n_steps", [(NV, 256, 16, 512, 2, 6, 2, 30), (F8, 256, 32, 512, 2, 70, 3, 16),
                                                      (NV, 2048, 256, 512, 8, 64, 4, 48)])
def test_cached_enqueue_prefetch(fmt, H, E, F, k, S, m, n_steps):
    L = Layer(fmt, H, E, F, cfg=71, layer=0, w_std=0.02)
    xs = ar1_states(0, 71, n_steps, H, [L.router], k + m)
    hp = L.host_pool()
    pool_res, R = torch.from_numpy(hp).cuda(), torch.from_numpy(np.ascontiguousarray(L.router)).cuda()
    host = torch.empty(E * L.stride, dtype=torch.uint8).pin_memory()
    host.numpy()[:] = hp
    slots = torch.zeros(S * L.stride, dtype=torch.uint8, device="cuda")
    cl = B.CachedLayer(R, host, slots, E, S, 1, k, rec_on_device=True)
    ws = torch.empty(B.moe_cached_layer_workspace(fmt, 1, H, F, k, E) + 256, dtype=torch.uint8, device="cuda")
    pf_buf = B.new_prefetch_buffer(E, k, m, S)
    pf_rec = B.prefetch_record(pf_buf, E, k, m, S)
    pf = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    eb = B.moe_expert_bytes(fmt, H, F)
    ref = olru.StampLRU(E, S)
    idx = torch.empty((1, k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, k), dtype=torch.float32, device="cuda")
    out = torch.empty((1, H), dtype=torch.uint16, device="cuda")
    pair_slot = torch.empty(k, dtype=torch.int32, device="cuda")
    pair_order = torch.empty(k, dtype=torch.int32, device="cuda")
    used = fetched = 0
    prev = set()
    for t in range(n_steps):
        xd = _x_dev(xs[t:t + 1])
        B.moe_cached_layer_enqueue_prefetch(fmt, L.stride, H, F, E, k, cl, xd, idx, w, pair_slot, pair_order, out,
                                            ws, m, pf_buf, pf)
        main.wait_stream(pf)
        idx_r, w_r, out_r = B.moe_layer_forward(fmt, pool_res, L.stride, H, F, E, k, xd, R)
        torch.cuda.synchronize()
        tag = f"step {t}"
        assert torch.equal(idx, idx_r) and torch.equal(w, w_r) and torch.equal(out, out_r), tag
        ranked = moe.route(xs[t:t + 1], L.router, k + m)[0][0]
        assert np.array_equal(idx.cpu().numpy()[0], ranked[:k]), tag
        r = ref.step(ranked[:k])
        rec = cl.miss_rec.cpu().numpy()
        assert rec[0] == 0 and (rec[1], rec[3]) == (r["n_miss"], r["n_hits"]), tag
        p = olru.prefetch_step(ref, ranked)
        prec = pf_rec.cpu().numpy()
        nm, n_max = int(p["n_miss"]), int(prec[4])
        assert prec[0] == 0 and prec[1] == nm, tag
        assert np.array_equal(prec[5:5 + nm], p["miss_expert"]), tag
        assert np.array_equal(prec[5 + n_max:5 + n_max + nm], p["miss_slot"]), tag
        assert np.array_equal(cl.lru.slot_expert.cpu().numpy(), ref.slot_expert), tag
        assert np.array_equal(cl.lru.slot_stamp.cpu().numpy(), ref.slot_stamp), tag
        assert int(cl.lru.clock.item()) == ref.clock, tag
        used += len(prev & set(int(e) for e in ranked[:k]))
        prev = set(int(e) for e in p["miss_expert"])
        fetched += len(prev)
        if t % 6 == 5 or t == n_steps - 1:
            for s_, e_ in enumerate(ref.slot_expert):
                if e_ >= 0:
                    assert np.array_equal(slots[s_ * L.stride:s_ * L.stride + eb].cpu().numpy(),
                                          hp[e_ * L.stride:e_ * L.stride + eb]), f"{tag} slot {s_}"
        if t == 0:
            o = moe.moe_layer(fmt, xs[:1], L.router, L.experts, k)
            assert_rows_close(bf16_dev_to_f64(out), fm.bf16_to_f64(o["out"]), what="out")
    assert fetched > 0 and 0 <= used <= fetched
