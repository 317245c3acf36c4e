"""GPU parity at the full sizes of the workloads that are timed.

* the 753B-class prefill (hidden 6144, 256 experts, top-8, width 2048, 4096
  tokens) in all three weight formats (MXFP4 on both of its grouped paths):
  routing of every token bit-exact, the per-pair ``y`` and the layer output of
  32 sampled tokens against the oracle;
* the cache-constrained decode at its real shape (hidden 2048, 256 experts,
  top-8, width 512, 64 VRAM slots per layer, NVFP4), two layers over 104
  AR(1) steps with an elastic resize to 96 slots on the way: at every step the
  device miss record, slot table, stamps and clock equal the oracle LRU and the
  output equals the all-resident layer bit for bit.

Sampled rows are chosen so that few distinct experts serve them (the oracle
dequantizes every expert it touches in fp64); the device pool holds those
experts' blobs and zero blobs elsewhere, which routes and schedules exactly
like full weights (routing reads only the router) and gives the other tokens
zero outputs.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from block_scaled_fp4_gemv_amd import binding as B  # noqa: E402
from oracle import formats as fm, lru as olru, moe  # noqa: E402

from helpers import Layer, ar1_states, assert_rows_close, bf16_dev_to_f64, iid_tokens  # noqa: E402

pytestmark = pytest.mark.gpu
NV, MX, F8 = 1, 2, 3


def _x_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def sample_rows(idx, n, E, seed):
    """n tokens whose routed experts overlap as much as possible: greedily the
    token adding the fewest experts not yet used (ties broken at random), first
    the last and the first token (the ragged tail and the head of every expert's
    row list)."""
    rng = np.random.default_rng(seed)
    T = idx.shape[0]
    have = np.zeros(E, bool)
    free = np.ones(T, bool)
    rows = []
    for t in (T - 1, 0):
        rows.append(t)
        free[t] = False
        have[idx[t]] = True
    while len(rows) < n:
        new = (~have[idx]).sum(axis=1)
        new[~free] = idx.shape[1] + 1
        cand = np.nonzero(new == new.min())[0]
        t = int(rng.choice(cand))
        rows.append(t)
        free[t] = False
        have[idx[t]] = True
    return np.array(sorted(rows))


@pytest.mark.parametrize("fmt", [NV, MX, F8])
def test_prefill_753b_shape_sampled(fmt):
    H, E, F, k, T = 6144, 256, 2048, 8, 4096
    L = Layer(fmt, H, E, F, cfg=4, layer=0, w_std=0.015, eager=False)
    x = iid_tokens(0, 4, T, H, [L.router], k)
    oidx, ow, _ = moe.route(x, L.router, k)
    rows = sample_rows(oidx, 32, E, seed=fmt)
    pool, R = L.device(needed=oidx[rows])
    xd = _x_dev(x)
    print(f"prefill753b fmt {fmt}: {len(np.unique(oidx[rows]))} experts serve the sampled rows", flush=True)
    ref = moe.moe_layer(fmt, x[rows], L.router, L.experts, k)
    # MXFP4 also on the native scaled MFMA (FP8 activation terms)
    for native in ((False, True) if fmt == MX else (False,)):
        idx, w, out = B.moe_layer_forward(fmt, pool, L.stride, H, F, E, k, xd, R,
                                          flags=B.MOE_LAYER_MX_NATIVE if native else 0)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), oidx)
        assert np.allclose(w.cpu().numpy(), ow, rtol=1e-3, atol=1e-7)
        idx2, w2, perm, off = B.moe_route(xd, R, k)
        y = torch.empty((T * k, H), dtype=torch.float32, device="cuda")
        B.moe_expert_ffn(fmt, pool, L.stride, H, F, E, xd, idx2, pair_perm=perm, expert_off=off, topk_w=w2, y=y,
                         flags=B.MOE_FFN_GROUPED | (B.MOE_FFN_MX_NATIVE if native else 0))
        torch.cuda.synchronize()
        assert torch.equal(idx2, idx)
        ysel = y.view(T, k, H)[torch.from_numpy(rows).cuda()].reshape(-1, H).cpu().numpy()
        del y
        assert_rows_close(ysel, ref["y"].reshape(-1, H), what=f"y native={native}")
        assert_rows_close(bf16_dev_to_f64(out)[rows], fm.bf16_to_f64(ref["out"]), what=f"out native={native}")


def _lru_state(st):
    return (st.slot_expert.cpu().numpy(), st.expert_slot.cpu().numpy(), st.slot_stamp.cpu().numpy(),
            int(st.clock.item()))


def test_cached_enqueue_cache35b_shape_with_resize():
    fmt, H, E, F, k, S = NV, 2048, 256, 512, 8, 64
    n_layers, n_steps, resize_at, S_new = 2, 104, 64, 96
    layers = [Layer(fmt, H, E, F, cfg=1, layer=l, w_std=0.02) for l in range(n_layers)]
    xs = ar1_states(0, 3, n_steps, H, [L.router for L in layers], k)
    eb = B.moe_expert_bytes(fmt, H, F)
    res, cls, hps, refs = [], [], [], []
    for L in layers:
        hp = L.host_pool()
        pool, R = torch.from_numpy(hp).cuda(), torch.from_numpy(np.ascontiguousarray(L.router)).cuda()
        host = torch.empty(E * L.stride, dtype=torch.uint8).pin_memory()
        host.numpy()[:] = hp
        slots = torch.zeros(S * L.stride, dtype=torch.uint8, device="cuda")
        res.append((pool, R))
        cls.append(B.CachedLayer(R, host, slots, E, S, 1, k, rec_on_device=True))
        hps.append(hp)
        refs.append(olru.StampLRU(E, S))
    ws = torch.empty(B.moe_cached_layer_workspace(fmt, 1, H, F, k, E) + 256, dtype=torch.uint8, device="cuda")
    idx = torch.empty((1, k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, k), dtype=torch.float32, device="cuda")
    out = torch.empty((1, H), dtype=torch.uint16, device="cuda")
    pair_slot = torch.empty(k, dtype=torch.int32, device="cuda")
    pair_order = torch.empty(k, dtype=torch.int32, device="cuda")

    def check_slots(l, what):
        se = refs[l].slot_expert
        pool = cls[l].slot_pool
        for s_, e_ in enumerate(se):
            if e_ >= 0:
                got = pool[s_ * layers[l].stride:s_ * layers[l].stride + eb].cpu().numpy()
                assert np.array_equal(got, hps[l][e_ * layers[l].stride:e_ * layers[l].stride + eb]), \
                    f"{what}: layer {l} slot {s_}"

    hits = acc = 0
    for t in range(n_steps):
        if t == resize_at:
            for l, cl in enumerate(cls):
                cl.resize(S_new, eb, layers[l].stride,
                          slot_pool=torch.zeros(S_new * layers[l].stride, dtype=torch.uint8, device="cuda"))
                refs[l].resize(S_new)
            torch.cuda.synchronize()
            for l in range(n_layers):
                assert [np.array_equal(a, b) for a, b in
                        zip(_lru_state(cls[l].lru)[:3], refs[l].state()[:3])] == [True] * 3, f"resize layer {l}"
                check_slots(l, "after resize")
        xd = _x_dev(xs[t:t + 1])
        for l, (L, cl) in enumerate(zip(layers, cls)):
            B.moe_cached_layer_enqueue(fmt, L.stride, H, F, E, k, cl, xd, idx, w, pair_slot, pair_order, out, ws)
            idx_r, w_r, out_r = B.moe_layer_forward(fmt, res[l][0], L.stride, H, F, E, k, xd, res[l][1])
            torch.cuda.synchronize()
            tag = f"step {t} layer {l}"
            assert torch.equal(idx, idx_r) and torch.equal(w, w_r), tag
            assert torch.equal(out, out_r), tag
            r = refs[l].step(idx.cpu().numpy().ravel())
            rec = cl.miss_rec.cpu().numpy()
            nm = int(r["n_miss"])
            n_max = int(rec[4])
            assert rec[0] == 0 and (rec[1], rec[2], rec[3]) == (nm, r["n_hit_pairs"], r["n_hits"]), tag
            assert np.array_equal(rec[5:5 + nm], r["miss_expert"]), tag
            assert np.array_equal(rec[5 + n_max:5 + n_max + nm], r["miss_slot"]), tag
            assert np.array_equal(pair_slot.cpu().numpy(), r["pair_slot"]), tag
            assert np.array_equal(pair_order.cpu().numpy(), r["pair_order"]), tag
            se, es, ss, clk = _lru_state(cl.lru)
            rse, res_, rss, rclk = refs[l].state()
            assert np.array_equal(se, rse) and np.array_equal(es, res_), tag
            assert np.array_equal(ss, rss) and clk == rclk, tag
            hits += r["n_hits"]
            acc += r["n_access"]
            if t == 0:
                ref = moe.moe_layer(fmt, xs[:1], L.router, L.experts, k)
                assert np.array_equal(idx.cpu().numpy(), ref["idx"]), tag
                assert_rows_close(bf16_dev_to_f64(out), fm.bf16_to_f64(ref["out"]), what="out")
    for l in range(n_layers):
        check_slots(l, "end")
    # the AR(1) states give the cache real reuse (neither all hits nor all misses)
    assert 0.3 < hits / acc < 0.98, hits / acc
