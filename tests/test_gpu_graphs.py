"""HIP graph replays against eager launches, in the configurations bench.py
times with graphs:

* the batch-1 decode stack (``bench.DecodeStack``: one moe_layer_forward per
  layer, each layer's down kernel reading the next router ahead, the whole
  step one graph) at the 35B shape in all three formats and at the 753B shape;
* the prefill layer (one graph per weight set, two weight sets replayed in
  turn, routers prepared once per set) at 2048 and 16384 tokens of the 35B
  shape in all three formats (MXFP4 on both grouped paths) and at 4096 tokens
  of the 753B shape;
* the cached decode step (moe_cached_layer_enqueue for every layer in one
  graph): per-layer caches, the runner-up prefetch on a second stream joined
  inside the graph, and one cache shared by a group of layers.

Each graph is replayed several times with new inputs, with eager launches of
the same entry points and host synchronisations between the replays, and every
replay must equal the eager result bit for bit: routing, outputs, miss and
prefetch records, LRU state and slot pools.  The eager paths are pinned to the
oracle by the parity tests; the first decode replay is also checked against it
here.
"""
import functools
import types

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import bench  # noqa: E402
from block_scaled_fp4_gemv_amd import binding as B  # noqa: E402
from block_scaled_fp4_gemv_amd import synth as sy  # noqa: E402
from oracle import formats as fm, lru as olru, moe  # noqa: E402

from helpers import Layer, ar1_states, assert_rows_close, bf16_dev_to_f64  # noqa: E402

pytestmark = pytest.mark.gpu
NV, MX, F8 = 1, 2, 3


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@functools.lru_cache(maxsize=None)
def _layer35(fmt, layer):
    """A seeded 35B-shape layer (hidden 2048, 256 experts, width 512), shared by the tests."""
    return Layer(fmt, 2048, 256, 512, cfg=31, layer=layer, w_std=0.02)


def _replicated_pool(fmt, H, E, F, cfg, copies):
    """Device pools of E blobs that all hold one seeded expert (its bytes, not
    zeros, so every routed pair computes), one independent copy per layer."""
    L = Layer(fmt, H, E, F, cfg=cfg, layer=0, w_std=0.015, eager=False)
    blob = _dev(L.blob(0))
    pool = torch.zeros(E * L.stride, dtype=torch.uint8, device="cuda")
    for e in range(E):
        pool[e * L.stride:e * L.stride + blob.numel()].copy_(blob)
    pools = [pool] + [pool.clone() for _ in range(copies - 1)]
    torch.cuda.synchronize()
    return pools, L.stride


def _check_stack_replays(stack, fmt, pools, routers, stride, H, F, E, k, n_replays, first=0):
    for i in range(first, first + n_replays):
        stack.replay(i)
        torch.cuda.synchronize()
        j = i % stack.n_states
        x = stack.xs_dev[j:j + 1]
        for l in range(stack.n_layers):
            idx, w, out = B.moe_layer_forward(fmt, pools[l], stride, H, F, E, k, x, routers[l])
            torch.cuda.synchronize()
            tag = f"replay {i} layer {l}"
            assert torch.equal(stack.idx[l], idx), tag
            assert torch.equal(stack.topk_w[l], w), tag
            assert torch.equal(stack.out[l], out), tag


@pytest.mark.parametrize("fmt,n_layers", [(NV, 4), (MX, 2), (F8, 2)])
def test_decode_stack_graph_35b_shape(fmt, n_layers):
    H, E, F, k = 2048, 256, 512, 8
    layers = [_layer35(fmt, l) for l in range(n_layers)]
    devs = [L.device() for L in layers]
    pools, routers = [d[0] for d in devs], [d[1] for d in devs]
    xs = ar1_states(0, 31, 8, H, [L.router for L in layers], k)
    wl = types.SimpleNamespace(H=H, E=E, F=F, k=k)
    stack = bench.DecodeStack(fmt, wl, pools, routers, layers[0].stride, n_layers, xs)
    # the first replay (state 0) against the oracle
    stack.replay(0)
    torch.cuda.synchronize()
    ref = moe.moe_layer(fmt, xs[:1], layers[0].router, layers[0].experts, k)
    assert np.array_equal(stack.idx[0].cpu().numpy(), ref["idx"])
    assert_rows_close(bf16_dev_to_f64(stack.out[0]), fm.bf16_to_f64(ref["out"]), what="out")
    _check_stack_replays(stack, fmt, pools, routers, layers[0].stride, H, F, E, k, n_replays=6, first=1)


@pytest.mark.parametrize("fmt", [NV, F8])
def test_decode_stack_graph_753b_shape(fmt):
    H, E, F, k, n_layers = 6144, 256, 2048, 8, 2
    pools, stride = _replicated_pool(fmt, H, E, F, cfg=32, copies=n_layers)
    routers = [_dev(sy.router(0, 32, l, E, H)) for l in range(n_layers)]
    xs = sy.ar1_sequence(0, 32, 6, H)
    wl = types.SimpleNamespace(H=H, E=E, F=F, k=k)
    stack = bench.DecodeStack(fmt, wl, pools, routers, stride, n_layers, xs)
    _check_stack_replays(stack, fmt, pools, routers, stride, H, F, E, k, n_replays=5)


def _check_prefill_replays(fmt, pools, Rs, stride, H, F, E, k, xs, flags=0):
    """Two weight sets, one graph each, captured as bench.py captures them; the
    replays alternate between the sets and take a new token batch each time."""
    T = xs[0].shape[0]
    Ps = [B.PreparedRouter(R) for R in Rs]
    x = torch.empty((T, H), dtype=torch.uint16, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H), dtype=torch.uint16, device="cuda")
    ws = B.new_layer_workspace(fmt, T, H, F, k, E)

    def run(l):
        B.moe_layer_forward(fmt, pools[l], stride, H, F, E, k, x, Ps[l], topk_idx=idx, topk_w=w, out=out, ws=ws,
                            flags=flags)

    x.copy_(xs[0])
    for l in (0, 1, 0):
        run(l)
    torch.cuda.synchronize()
    graphs = []
    for l in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run(l)
        graphs.append(g)
    torch.cuda.synchronize()
    for r in range(len(xs)):
        l = r % 2
        x.copy_(xs[r])
        graphs[l].replay()
        torch.cuda.synchronize()
        idx_e, w_e, out_e = B.moe_layer_forward(fmt, pools[l], stride, H, F, E, k, xs[r], Ps[l], flags=flags)
        torch.cuda.synchronize()
        tag = f"replay {r} weight set {l}"
        assert torch.equal(idx, idx_e), tag
        assert torch.equal(w, w_e), tag
        assert torch.equal(out, out_e), tag


@pytest.mark.parametrize("fmt,T,flags", [(NV, 2048, 0), (MX, 2048, 0), (MX, 2048, B.MOE_LAYER_MX_NATIVE),
                                         (F8, 2048, 0), (NV, 16384, 0)])
def test_prefill_graph_35b_shape(fmt, T, flags):
    H, E, F, k = 2048, 256, 512, 8
    layers = [_layer35(fmt, l) for l in range(2)]
    devs = [L.device() for L in layers]
    xs = [_dev(sy.token_rows(0, 33 + r, T, H)) for r in range(4)]
    _check_prefill_replays(fmt, [d[0] for d in devs], [d[1] for d in devs], layers[0].stride, H, F, E, k, xs,
                           flags=flags)


def test_prefill_graph_753b_shape():
    fmt, H, E, F, k, T = NV, 6144, 256, 2048, 8, 4096
    pools, stride = _replicated_pool(fmt, H, E, F, cfg=34, copies=2)
    Rs = [_dev(sy.router(0, 34, l, E, H)) for l in range(2)]
    xs = [_dev(sy.token_rows(0, 34 + r, T, H)) for r in range(3)]
    _check_prefill_replays(fmt, pools, Rs, stride, H, F, E, k, xs)


class _CachedStep:
    """One executor of the cached decode step over a stack of layers: its own
    caches, LRU states, records and per-layer outputs.  kind: "plain" (a cache
    per layer), "prefetch" (runner-up prefetch of m experts on a second stream,
    forked and joined inside the step) or "shared" (one cache for all layers,
    keyed by layer)."""

    def __init__(self, kind, fmt, H, E, F, k, S, m, hosts, routers, stride):
        self.kind, self.fmt, self.H, self.E, self.F, self.k, self.m = kind, fmt, H, E, F, k, m
        self.stride = stride
        n = len(hosts)
        if kind == "shared":
            self.state = B.LRUState(n * E, n * S)
            B.moe_lru_reset(self.state)
            pool = torch.zeros(n * S * stride, dtype=torch.uint8, device="cuda")
            self.layers = [B.CachedLayer(routers[j], hosts[j], pool, E, n * S, 1, k, rec_on_device=True,
                                         lru=self.state.view(j * E)) for j in range(n)]
            self.states = [self.state]
        else:
            self.layers = [B.CachedLayer(routers[j], hosts[j],
                                         torch.zeros(S * stride, dtype=torch.uint8, device="cuda"),
                                         E, S, 1, k, rec_on_device=True) for j in range(n)]
            self.states = [L.lru for L in self.layers]
        self.ws = torch.empty(B.moe_cached_layer_workspace(fmt, 1, H, F, k, E) + 256, dtype=torch.uint8,
                              device="cuda")
        self.x = torch.empty((1, H), dtype=torch.uint16, device="cuda")
        self.idx = [torch.empty((1, k), dtype=torch.int32, device="cuda") for _ in range(n)]
        self.w = [torch.empty((1, k), dtype=torch.float32, device="cuda") for _ in range(n)]
        self.out = [torch.empty((1, H), dtype=torch.uint16, device="cuda") for _ in range(n)]
        self.pair_slot = [torch.empty(k, dtype=torch.int32, device="cuda") for _ in range(n)]
        self.pair_order = [torch.empty(k, dtype=torch.int32, device="cuda") for _ in range(n)]
        if kind == "prefetch":
            self.pf = torch.cuda.Stream()
            self.bufs = [B.new_prefetch_buffer(E, k, m, S) for _ in range(n)]
            self.precs = [B.prefetch_record(b, E, k, m, S) for b in self.bufs]
        self.graph = None

    def enqueue(self):
        main = torch.cuda.current_stream()
        if self.kind == "prefetch":
            self.pf.wait_stream(main)
        for j, L in enumerate(self.layers):
            args = (self.fmt, self.stride, self.H, self.F, self.E, self.k, L, self.x, self.idx[j], self.w[j],
                    self.pair_slot[j], self.pair_order[j], self.out[j], self.ws)
            if self.kind == "prefetch":
                B.moe_cached_layer_enqueue_prefetch(*args, self.m, self.bufs[j], self.pf)
            else:
                B.moe_cached_layer_enqueue(*args)
        if self.kind == "prefetch":
            main.wait_stream(self.pf)

    def capture(self):
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.enqueue()
        torch.cuda.synchronize()

    def step(self, x):
        self.x.copy_(x)
        if self.graph is None:
            self.enqueue()
        else:
            self.graph.replay()

    def snapshot(self):
        """Everything the step defines, on the host."""
        snap = {}
        for j, L in enumerate(self.layers):
            for name in ("idx", "w", "out", "pair_slot", "pair_order"):
                snap[f"{name}{j}"] = getattr(self, name)[j].cpu().numpy()
            recs = [("rec", L.miss_rec)] + ([("prefetch_rec", self.precs[j])] if self.kind == "prefetch" else [])
            for name, r in recs:
                r = r.cpu().numpy()
                nm, n_max = int(r[1]), int(r[4])
                snap[f"{name}{j}"] = np.concatenate([r[:5], r[5:5 + nm], r[5 + n_max:5 + n_max + nm]])
        for j, st in enumerate(self.states):
            for name in ("slot_expert", "expert_slot", "slot_stamp", "clock"):
                snap[f"{name}{j}"] = getattr(st, name).cpu().numpy()
        return snap

    def pools_equal(self, other):
        return all(torch.equal(a.slot_pool, b.slot_pool) for a, b in zip(self.layers, other.layers))


@pytest.mark.parametrize("kind", ["plain", "prefetch", "shared"])
def test_cached_step_graph_cache35b_shape(kind):
    fmt, H, E, F, k, S, m = NV, 2048, 256, 512, 8, 64, 2
    n_layers, warm, n_steps = 2, 4, 24
    layers = [_layer35(fmt, l) for l in range(n_layers)]
    stride = layers[0].stride
    hosts, routers = [], []
    for L in layers:
        h = torch.empty(E * stride, dtype=torch.uint8).pin_memory()
        L.host_pool(out=h.numpy())
        hosts.append(h)
        routers.append(_dev(L.router))
    xs = _dev(ar1_states(0, 35, warm + n_steps, H, [L.router for L in layers], k + m))
    g = _CachedStep(kind, fmt, H, E, F, k, S, m, hosts, routers, stride)
    e = _CachedStep(kind, fmt, H, E, F, k, S, m, hosts, routers, stride)
    refs = [olru.StampLRU(E, S) for _ in range(n_layers)] if kind == "plain" else None
    for t in range(warm):
        for ex in (g, e):
            ex.step(xs[t:t + 1])
        if refs:
            torch.cuda.synchronize()
            for j in range(n_layers):
                refs[j].step(g.idx[j].cpu().numpy().ravel())
    g.capture()
    misses = 0
    for t in range(warm, warm + n_steps):
        g.step(xs[t:t + 1])
        torch.cuda.synchronize()
        e.step(xs[t:t + 1])
        torch.cuda.synchronize()
        a, b = g.snapshot(), e.snapshot()
        assert a.keys() == b.keys()
        for key in a:
            assert np.array_equal(a[key], b[key]), f"step {t}: {key}"
        assert g.pools_equal(e), f"step {t}: slot pools"
        for j in range(n_layers):
            assert a[f"rec{j}"][0] == 0, f"step {t}: capacity error"
            misses += int(a[f"rec{j}"][1])
            if refs:
                r = refs[j].step(a[f"idx{j}"].ravel())
                assert int(a[f"rec{j}"][1]) == r["n_miss"], f"step {t} layer {j}"
                assert np.array_equal(a[f"slot_expert{j}"], refs[j].slot_expert), f"step {t} layer {j}"
                assert np.array_equal(a[f"slot_stamp{j}"], refs[j].slot_stamp), f"step {t} layer {j}"
    assert misses > 0
