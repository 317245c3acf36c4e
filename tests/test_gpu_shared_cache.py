"""GPU parity of the expert cache shared by several layers (one keyed LRU state
and one slot pool; layer j's expert e is key j*E + e).

Every layer step through moe_cached_layer_enqueue (or moe_cache_lookup) must
give the oracle's shared-cache records, slot table, stamps and clock
(oracle.lru.LayerView over StampLRU), outputs equal to the all-resident layer
bit for bit, and slots holding the host blobs of the (layer, expert) they name.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from block_scaled_fp4_gemv_amd import binding as B  # noqa: E402
from oracle import formats as fm, lru as olru, moe  # noqa: E402

from helpers import Layer, ar1_states, assert_rows_close, bf16_dev_to_f64  # noqa: E402

pytestmark = pytest.mark.gpu
NV, MX = 1, 2


def _x_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _run_shared(fmt, H, E, F, k, S, T, n_layers, n_steps, cfg, oracle_step0=True):
    layers = [Layer(fmt, H, E, F, cfg=cfg, layer=j, w_std=0.02) for j in range(n_layers)]
    xs = ar1_states(0, cfg, n_steps * T, H, [L.router for L in layers], k)
    eb = B.moe_expert_bytes(fmt, H, F)
    stride = layers[0].stride
    state = B.LRUState(n_layers * E, S)
    B.moe_lru_reset(state)
    pool = torch.zeros(S * stride, dtype=torch.uint8, device="cuda")
    ref = olru.StampLRU(n_layers * E, S)
    views = [olru.LayerView(ref, j * E) for j in range(n_layers)]
    cls, res, hps = [], [], []
    for j, L in enumerate(layers):
        hp = L.host_pool()
        host = torch.empty(E * stride, dtype=torch.uint8).pin_memory()
        host.numpy()[:] = hp
        R = torch.from_numpy(np.ascontiguousarray(L.router)).cuda()
        cls.append(B.CachedLayer(R, host, pool, E, S, T, k, rec_on_device=True, lru=state.view(j * E)))
        res.append((torch.from_numpy(hp).cuda(), R))
        hps.append(hp)
    ws = torch.empty(B.moe_cached_layer_workspace(fmt, T, H, F, k, E) + 256, dtype=torch.uint8, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H), dtype=torch.uint16, device="cuda")
    pair_slot = torch.empty(T * k, dtype=torch.int32, device="cuda")
    pair_order = torch.empty(T * k, dtype=torch.int32, device="cuda")
    hits = acc = 0
    for t in range(n_steps):
        xd = _x_dev(xs[t * T:(t + 1) * T])
        for j, (L, cl) in enumerate(zip(layers, cls)):
            B.moe_cached_layer_enqueue(fmt, stride, H, F, E, k, cl, xd, idx, w, pair_slot, pair_order, out, ws)
            idx_r, w_r, out_r = B.moe_layer_forward(fmt, res[j][0], stride, H, F, E, k, xd, res[j][1])
            torch.cuda.synchronize()
            tag = f"step {t} layer {j}"
            assert torch.equal(idx, idx_r) and torch.equal(w, w_r) and torch.equal(out, out_r), tag
            r = views[j].step(idx.cpu().numpy().ravel())
            rec = cl.miss_rec.cpu().numpy()
            nm, n_max = int(r["n_miss"]), int(rec[4])
            assert rec[0] == 0 and (rec[1], rec[2], rec[3]) == (nm, r["n_hit_pairs"], r["n_hits"]), tag
            assert np.array_equal(rec[5:5 + nm], r["miss_expert"]), tag
            assert np.array_equal(rec[5 + n_max:5 + n_max + nm], r["miss_slot"]), tag
            assert np.array_equal(pair_slot.cpu().numpy(), r["pair_slot"]), tag
            assert np.array_equal(pair_order.cpu().numpy(), r["pair_order"]), tag
            assert np.array_equal(state.slot_expert.cpu().numpy(), ref.slot_expert), tag
            assert np.array_equal(state.expert_slot.cpu().numpy(), ref.expert_slot), tag
            assert np.array_equal(state.slot_stamp.cpu().numpy(), ref.slot_stamp), tag
            assert int(state.clock.item()) == ref.clock, tag
            hits += r["n_hits"]
            acc += r["n_access"]
            if t == 0 and j == 0 and oracle_step0:
                o = moe.moe_layer(fmt, xs[:T], L.router, L.experts, k)
                assert np.array_equal(idx.cpu().numpy(), o["idx"])
                assert_rows_close(bf16_dev_to_f64(out), fm.bf16_to_f64(o["out"]), what="out")
        if t % 8 == 7 or t == n_steps - 1:
            for s_, key in enumerate(ref.slot_expert):
                if key >= 0:
                    j, e = divmod(int(key), E)
                    got = pool[s_ * stride:s_ * stride + eb].cpu().numpy()
                    assert np.array_equal(got, hps[j][e * stride:e * stride + eb]), f"step {t} slot {s_}"
    return hits / acc


@pytest.mark.parametrize("S,T", [(10, 1), (72, 1), (12, 3)])
def test_shared_cache_small(S, T):
    """Three layers (16 experts each, top-2) on one cache: 10 slots (one-wave
    lookup with the top-k fused), 72 slots (workgroup lookup), 3 tokens per step."""
    _run_shared(NV, 256, 16, 512, 2, S, T, n_layers=3, n_steps=24 if T == 1 else 10, cfg=61)


def test_shared_cache_35b_shape():
    """Four 35B-shape layers (256 experts, top-8, NVFP4) sharing 256 slots
    (1024 keys: the workgroup lookup at its key limit), 24 AR(1) steps."""
    rate = _run_shared(NV, 2048, 256, 512, 8, 256, 1, n_layers=4, n_steps=24, cfg=62, oracle_step0=True)
    assert 0.2 < rate < 0.99, rate


def test_shared_cache_lookup_call():
    """moe_cache_lookup on keyed views of one state: two layers' experts as
    keys 0.. and 20.., records in experts, state equal to the oracle."""
    E, S, k = 20, 7, 3
    state = B.LRUState(2 * E, S)
    B.moe_lru_reset(state)
    ref = olru.StampLRU(2 * E, S)
    views = [olru.LayerView(ref, 0), olru.LayerView(ref, E)]
    rng = np.random.default_rng(9)
    rec = torch.zeros(B.moe_miss_record_words(1, k, S), dtype=torch.int32, device="cuda")
    pair_slot = torch.empty(k, dtype=torch.int32, device="cuda")
    pair_order = torch.empty(k, dtype=torch.int32, device="cuda")
    for t in range(40):
        j = t % 2
        acc = rng.choice(8 + 4 * j, size=k, replace=False).astype(np.int32)
        B.moe_cache_lookup(state.view(j * E), torch.from_numpy(acc).cuda().view(1, k), pair_slot, pair_order, rec)
        torch.cuda.synchronize()
        r = views[j].step(acc)
        got = rec.cpu().numpy()
        nm = int(r["n_miss"])
        assert got[0] == 0 and got[1] == nm and np.array_equal(got[5:5 + nm], r["miss_expert"])
        assert np.array_equal(pair_slot.cpu().numpy(), r["pair_slot"])
        assert np.array_equal(state.slot_expert.cpu().numpy(), ref.slot_expert)
