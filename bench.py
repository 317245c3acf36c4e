#!/usr/bin/env python3
"""Benchmark: routed block-scaled MoE layer stack, batch-1 decode, one MI355X.

Workload (default): the 35B-A3B-like decode stack - 40 MoE layers, hidden 2048,
256 experts, top-8, expert width 512, NVFP4 weights drawn from N(0, 0.02),
fp32 router N(0, 0.05), batch 1, AR(1) bf16 hidden states
h_t = 0.9 h_{t-1} + 0.44 eps_t.  Every layer of a step receives the same h_t.
A step is one token through the whole stack: per layer one moe_layer_forward
call (router GEMV, softmax + top-8, gate/up + SwiGLU, down, gate-weighted
combine) through the C ABI, layers in order, the step captured in one HIP graph.  All
weights are resident in HBM before timing starts.

Prints one JSON line (rank 0): tok/s, ms/step, the dominant kernel's roofline
(HIP-event timed inside the timed region), and the CPU oracle timed on a
bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "MoE-layer decode tok/s + weight-stream HBM GB/s; prefill MFMA util (1 GPU)"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode35b", choices=["decode35b", "decode753b"])
    p.add_argument("--prefill", default="prefill35b", choices=["prefill35b", "prefill35b_16k", "prefill753b", "none"],
                   help="prefill workload timed alongside the decode headline")
    p.add_argument("--prefill-reps", type=int, default=20)
    p.add_argument("--compute-bound-reps", type=int, default=10,
                   help="with --prefill prefill35b: also time the same layer at 16384 tokens, the compute-bound "
                        "point (0 = skip)")
    p.add_argument("--cache", default="cache35b", choices=["cache35b", "none"],
                   help="cache-constrained decode timed on the same layers (VRAM slot pools + pinned host pools)")
    p.add_argument("--cache-warmup", type=int, default=64)
    p.add_argument("--no-read-ahead", action="store_true",
                   help="plain moe_layer_forward per decode layer (no warming of the next router)")
    p.add_argument("--cache-steps", type=int, default=128)
    p.add_argument("--cache-elastic-steps", type=int, default=64,
                   help="after the timed cache steps: resize every layer's slot cache (half in place, then "
                        "1.5x into new pools) and run this many steps after each resize (0 = skip)")
    p.add_argument("--cache-split-steps", type=int, default=48,
                   help="timed steps of each q run of the GPU-fill / CPU-expert miss split (0 = skip)")
    p.add_argument("--cache-split-warmup", type=int, default=24)
    p.add_argument("--cache-prefetch-steps", type=int, default=96,
                   help="steps of each runner-up prefetch run on the cache workload (m = 2, 4; 0 = skip)")
    p.add_argument("--cache-shared-steps", type=int, default=96,
                   help="steps of the cross-layer cache comparison (per-layer vs shared pools on a trace with "
                        "unequal demand; 0 = skip)")
    p.add_argument("--cache-host-sync", action="store_true",
                   help="time the host-waiting executor (moe_cached_layer_forward) instead")
    p.add_argument("--prefill-stream-reps", type=int, default=3,
                   help="streamed-prefill leg passes (0 = skip; runs with the cache leg's host pools)")
    p.add_argument("--fmt", type=int, default=0, help="override weight format (1 NVFP4, 2 MXFP4, 3 FP8)")
    p.add_argument("--plain-router", action="store_true",
                   help="prefill legs: pass the fp32 router (split into bf16 planes on every call) instead of a "
                        "router prepared once per weight set")
    p.add_argument("--mx-native", action="store_true",
                   help="MXFP4 prefill on the native scaled MFMA (FP4 weights x two FP8 activation terms) instead "
                        "of bf16 MFMA with the weights dequantized in registers")
    p.add_argument("--layers", type=int, default=0, help="override the layer count (testing only)")
    p.add_argument("--replicate-layers", action="store_true",
                   help="generate layer 0's experts once and give every other layer its own device copy "
                        "(distinct addresses, same bytes; routers stay per layer) - for the large stacks")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--c4-steps", type=int, default=100,
                   help="timed decode steps of the 753B-class stack leg (0 = skip the leg)")
    p.add_argument("--c4-prefill-reps", type=int, default=5,
                   help="passes of the 753B-class 4096-token prefill in that leg (0 = skip)")
    p.add_argument("--c4-cpu", type=int, default=8,
                   help="753B-class leg: time the oracle on one decode token and on this many prefill tokens "
                        "(0 = skip)")
    p.add_argument("--cpu-prefill-tokens", type=int, default=512,
                   help="time the oracle on this many tokens of the prefill leg's input (0 = skip)")
    p.add_argument("--persistence-steps", type=int, default=32,
                   help="decode steps after the timed ones over which the previous step's routing is compared "
                        "with each step's (0 = skip)")
    p.add_argument("--cpu-sample-steps", type=int, default=6)
    p.add_argument("--threads", type=int, default=min(16, os.cpu_count() or 1))
    p.add_argument("--calib-copy-mib", type=int, default=256,
                   help="one device-to-device copy of this size before timing: a kernel of known "
                        "traffic for scaling hardware byte counters (0 = skip)")
    return p.parse_args()


def build_stack(wl, fmt, n_layers, threads, keep_host=False, replicate=False, batch0=None):
    """Generate, quantize, pack and upload every layer; returns device pools, routers,
    the blob stride and (keep_host) the pinned host copy of every layer.  With
    replicate, layers after the first get a device copy of layer 0's experts.  A
    list passed as batch0 receives layer 0's canonical experts (for the oracle)."""
    import torch

    from block_scaled_fp4_gemv_amd import binding as B
    from block_scaled_fp4_gemv_amd import synth as sy

    sy.set_threads(threads)
    stride = B.blob_stride(fmt, wl.H, wl.F)
    pools, routers, hosts = [], [], []
    host = torch.empty(wl.E * stride, dtype=torch.uint8).pin_memory()
    t0 = time.time()
    for l in range(n_layers):
        if replicate and l > 0:
            pools.append(pools[0].clone())
            routers.append(torch.from_numpy(sy.router(0, wl.wcfg, l, wl.E, wl.H)).cuda())
            continue
        batch = sy.experts(fmt, 0, wl.wcfg, l, 0, wl.E, wl.H, wl.F, wl.w_std)
        if batch0 is not None and l == 0:
            batch0.append(batch)
        if keep_host and l > 0:
            host = torch.empty(wl.E * stride, dtype=torch.uint8).pin_memory()
        B.pack_layer(fmt, wl.H, wl.F, batch, host.numpy(), stride, threads=threads)
        del batch
        pools.append(host.cuda())
        if keep_host:
            hosts.append(host)
        routers.append(torch.from_numpy(sy.router(0, wl.wcfg, l, wl.E, wl.H)).cuda())
        if l % 4 == 3 or l == n_layers - 1:
            log(f"layer {l + 1}/{n_layers} generated ({time.time() - t0:.0f} s)")
    torch.cuda.synchronize()
    return pools, routers, stride, hosts


def cache_leg(name, fmt, hosts, routers, stride, warmup, steps, host_sync=False, elastic_steps=0):
    """Cache-constrained decode: each layer keeps S of its E experts in a VRAM slot
    pool.  Default: moe_cached_layer_enqueue per layer on one stream (router, LRU
    lookup, every pair's experts with the misses streamed from the pinned host
    pool into their slots, combine; nothing waits on the host).  host_sync: the
    moe_cached_layer_forward executor (host wait on every layer's miss record,
    one hipMemcpyAsync per miss)."""
    import numpy as np
    import torch

    from block_scaled_fp4_gemv_amd import binding as B
    from block_scaled_fp4_gemv_amd import synth as sy

    wl = sy.WORKLOADS[name]
    H, E, F, k, S = wl.H, wl.E, wl.F, wl.k, wl.slots
    n_layers = len(hosts)
    layers = [B.CachedLayer(routers[l], hosts[l], torch.zeros(S * stride, dtype=torch.uint8, device="cuda"),
                            E, S, 1, k, rec_on_device=not host_sync) for l in range(n_layers)]
    ws = torch.empty(B.moe_cached_layer_workspace(fmt, 1, H, F, k, E) + 256, dtype=torch.uint8, device="cuda")
    n_el = 0 if host_sync else 2 * elastic_steps
    xs = torch.from_numpy(sy.ar1_sequence(0, wl.cfg_id, warmup + steps + n_el, H)).cuda()
    idx = torch.empty((1, k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, k), dtype=torch.float32, device="cuda")
    pair_slot = torch.empty(k, dtype=torch.int32, device="cuda")
    pair_order = torch.empty(k, dtype=torch.int32, device="cuda")
    out = torch.empty((1, H), dtype=torch.uint16, device="cuda")
    copy = torch.cuda.Stream()
    eb = B.moe_expert_bytes(fmt, H, F)
    recs = []

    xbuf = torch.empty((1, H), dtype=torch.uint16, device="cuda")
    graph = [None]

    def enqueue_layers():
        for L in layers:
            B.moe_cached_layer_enqueue(fmt, stride, H, F, E, k, L, xbuf, idx, w, pair_slot, pair_order, out, ws)

    def step(t):
        x = xs[t:t + 1]
        if host_sync:
            hm = np.zeros(2, np.int64)
            for L in layers:
                hm += B.moe_cached_layer_forward(fmt, stride, H, F, E, k, L, x, idx, w, pair_slot, pair_order,
                                                 out, ws, copy_stream=copy)
            recs.append(hm)
        else:
            xbuf.copy_(x)
            if graph[0] is None:
                enqueue_layers()
            else:
                graph[0].replay()
            recs.append(torch.stack([L.miss_rec[:4] for L in layers]))

    for t in range(warmup):
        step(t)
    torch.cuda.synchronize()
    if not host_sync:
        # the whole 40-layer step on one stream: capture it once, replay per token
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            enqueue_layers()
        torch.cuda.synchronize()
        graph[0] = g
    recs.clear()
    t0 = time.perf_counter()
    for t in range(warmup, warmup + steps):
        step(t)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    if host_sync:
        tot = np.sum(recs, axis=0)
    else:
        r = torch.stack(recs).cpu().numpy()
        assert (r[:, :, 0] == 0).all(), "cache capacity error"
        tot = np.array([r[:, :, 3].sum(), r[:, :, 1].sum()], np.int64)
    acc = steps * n_layers * k
    elastic = []
    if n_el:
        # elastic slot pools: halve every layer's cache in place, then grow it to
        # 1.5x into new pools; each resize is timed with events, and the decode
        # steps that follow it run from a newly captured graph
        t = warmup + steps
        for S_new, in_place in ((S // 2, True), (S + S // 2, False)):
            wsz = B.moe_lru_resize_workspace(S_new)
            wsr = torch.empty(n_layers * wsz, dtype=torch.uint8, device="cuda")
            pools = [None if in_place else torch.zeros(S_new * stride, dtype=torch.uint8, device="cuda")
                     for _ in layers]
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i, L in enumerate(layers):
                L.resize(S_new, eb, stride, slot_pool=pools[i], ws=wsr[i * wsz:(i + 1) * wsz])
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            copied = int(wsr.view(torch.int32).reshape(n_layers, -1)[:, 0].sum().item())
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                enqueue_layers()
            torch.cuda.synchronize()
            graph[0] = g
            recs.clear()
            t0 = time.perf_counter()
            for _ in range(elastic_steps):
                step(t)
                t += 1
            torch.cuda.synchronize()
            dte = time.perf_counter() - t0
            r = torch.stack(recs).cpu().numpy()
            assert (r[:, :, 0] == 0).all(), "cache capacity error"
            elastic.append({"slots": S_new, "pool": "rebuilt in place" if in_place else "new pools",
                            "resize_ms_all_layers": round(ms, 3), "blobs_copied": copied,
                            "copy_GBps": round(copied * eb / (ms * 1e-3) / 1e9, 1) if ms > 0 else None,
                            "steps_after": elastic_steps, "tokens_per_s": round(elastic_steps / dte, 2),
                            "hit_rate": round(float(r[:, :, 3].sum()) / (elastic_steps * n_layers * k), 4),
                            "misses_per_token": round(float(r[:, :, 1].sum()) / elastic_steps, 2)})
    return {"workload": f"{name}: {n_layers} layers, hidden {H}, {E} experts, top-{k}, width {F}, "
                        f"{S} VRAM slots per layer, batch 1, pinned host pool",
            "executor": "moe_cached_layer_forward (host waits per layer)" if host_sync else
                        "moe_cached_layer_enqueue x 40 layers captured in one HIP graph (one stream; misses "
                        "streamed from the host pool into their slots)",
            "tokens_per_s": round(steps / dt, 2), "ms_per_step": round(dt / steps * 1e3, 3),
            "warmup_steps": warmup, "timed_steps": steps, "hit_rate": round(float(tot[0]) / acc, 4),
            "misses_per_token": round(float(tot[1]) / steps, 2),
            "h2d_GBps": round(float(tot[1]) * eb / dt / 1e9, 2), "expert_blob_bytes": eb,
            "timing": "host wall clock over the timed steps, synchronised at both ends",
            **({"elastic": elastic} if elastic else {})}


def cache_shared_leg(fmt, hosts, stride, warmup, steps, group=4):
    """The global cache in its cross-layer form: the decode35b layers with routers
    whose rows are scaled by exp(sigma * N(0,1)), sigma = layer % 4 (unequal
    demand: larger sigma concentrates routing on fewer experts), run once with a
    64-slot cache per layer and once with one 256-slot cache shared by each group
    of 4 layers (the same slots in all).  Each 40-layer step is one HIP graph."""
    import numpy as np
    import torch

    from block_scaled_fp4_gemv_amd import binding as B
    from block_scaled_fp4_gemv_amd import synth as sy

    wl = sy.WORKLOADS["cache35b"]
    H, E, F, k, S = wl.H, wl.E, wl.F, wl.k, wl.slots
    n_layers = len(hosts)
    routers = [torch.from_numpy(sy.router_skewed(0, wl.wcfg, l, E, H, float(l % group))).cuda()
               for l in range(n_layers)]
    xs = torch.from_numpy(sy.ar1_sequence(0, wl.cfg_id, warmup + steps, H)).cuda()
    ws = torch.empty(B.moe_cached_layer_workspace(fmt, 1, H, F, k, E) + 256, dtype=torch.uint8, device="cuda")
    idx = torch.empty((1, k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, k), dtype=torch.float32, device="cuda")
    pair_slot = torch.empty(k, dtype=torch.int32, device="cuda")
    pair_order = torch.empty(k, dtype=torch.int32, device="cuda")
    out = torch.empty((1, H), dtype=torch.uint16, device="cuda")
    xbuf = torch.empty((1, H), dtype=torch.uint16, device="cuda")
    eb = B.moe_expert_bytes(fmt, H, F)
    res = {}
    for mode in ("per_layer", "shared"):
        layers = []
        if mode == "per_layer":
            for l in range(n_layers):
                pool = torch.zeros(S * stride, dtype=torch.uint8, device="cuda")
                layers.append(B.CachedLayer(routers[l], hosts[l], pool, E, S, 1, k, rec_on_device=True))
        else:
            for g in range(0, n_layers, group):
                n = min(group, n_layers - g)
                state = B.LRUState(n * E, n * S)
                B.moe_lru_reset(state)
                pool = torch.zeros(n * S * stride, dtype=torch.uint8, device="cuda")
                for j in range(n):
                    layers.append(B.CachedLayer(routers[g + j], hosts[g + j], pool, E, n * S, 1, k,
                                                rec_on_device=True, lru=state.view(j * E)))

        def enqueue():
            for L in layers:
                B.moe_cached_layer_enqueue(fmt, stride, H, F, E, k, L, xbuf, idx, w, pair_slot, pair_order, out, ws)

        for t in range(warmup):
            xbuf.copy_(xs[t:t + 1])
            enqueue()
        torch.cuda.synchronize()
        g_ = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_):
            enqueue()
        torch.cuda.synchronize()
        recs = []
        t0 = time.perf_counter()
        for t in range(warmup, warmup + steps):
            xbuf.copy_(xs[t:t + 1])
            g_.replay()
            recs.append(torch.stack([L.miss_rec[:4] for L in layers]))
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        r = torch.stack(recs).cpu().numpy()
        assert (r[:, :, 0] == 0).all(), "cache capacity error"
        hits, misses = float(r[:, :, 3].sum()), float(r[:, :, 1].sum())
        res[mode] = {"slots": f"{S} per layer" if mode == "per_layer" else f"{group * S} per group of {group} layers",
                     "tokens_per_s": round(steps / dt, 2), "hit_rate": round(hits / (steps * n_layers * k), 4),
                     "misses_per_token": round(misses / steps, 2),
                     "h2d_GBps": round(misses * eb / dt / 1e9, 2)}
        del layers
        torch.cuda.empty_cache()
    return {"workload": f"cache35b layers with unequal demand (router rows scaled by exp(sigma * N(0,1)), sigma = "
                        f"layer % {group}), {n_layers} layers, batch 1",
            "warmup_steps": warmup, "timed_steps": steps, **res,
            "miss_reduction": round(1 - res["shared"]["misses_per_token"] /
                                    max(res["per_layer"]["misses_per_token"], 1e-9), 4)}


def cache_prefetch_leg(fmt, hosts, routers, stride, warmup, steps, ms=(2, 4)):
    """Predictive prefetch on the cache35b decode (moe_cached_layer_enqueue_prefetch):
    for each m, the 40-layer step with every layer's runner-up experts (ranks
    k..k+m-1) prefetched on a second stream (one HIP graph per step, the
    prefetch stream joined at its end).  Reports tok/s, the routed hit rate,
    blobs moved over PCIe per token (routed misses + prefetches) and prefetch
    accuracy: the share of prefetched experts that the same layer routes to at
    the next step."""
    import numpy as np
    import torch

    from block_scaled_fp4_gemv_amd import binding as B
    from block_scaled_fp4_gemv_amd import synth as sy

    wl = sy.WORKLOADS["cache35b"]
    H, E, F, k, S = wl.H, wl.E, wl.F, wl.k, wl.slots
    n_layers = len(hosts)
    xs = torch.from_numpy(sy.ar1_sequence(0, wl.cfg_id, warmup + steps, H)).cuda()
    ws = torch.empty(B.moe_cached_layer_workspace(fmt, 1, H, F, k, E) + 256, dtype=torch.uint8, device="cuda")
    idx = torch.empty((n_layers, 1, k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, k), dtype=torch.float32, device="cuda")
    pair_slot = torch.empty(k, dtype=torch.int32, device="cuda")
    pair_order = torch.empty(k, dtype=torch.int32, device="cuda")
    out = torch.empty((1, H), dtype=torch.uint16, device="cuda")
    xbuf = torch.empty((1, H), dtype=torch.uint16, device="cuda")
    eb = B.moe_expert_bytes(fmt, H, F)
    pf = torch.cuda.Stream()
    runs = []
    for m in ms:
        layers = [B.CachedLayer(routers[l], hosts[l], torch.zeros(S * stride, dtype=torch.uint8, device="cuda"),
                                E, S, 1, k, rec_on_device=True) for l in range(n_layers)]
        bufs = [B.new_prefetch_buffer(E, k, m, S) for _ in range(n_layers)]
        precs = [B.prefetch_record(b, E, k, m, S) for b in bufs]
        nw = B.moe_miss_record_words(1, k + m, S)

        def enqueue():
            main = torch.cuda.current_stream()
            pf.wait_stream(main)
            for l, L in enumerate(layers):
                B.moe_cached_layer_enqueue_prefetch(fmt, stride, H, F, E, k, L, xbuf, idx[l], w, pair_slot,
                                                    pair_order, out, ws, m, bufs[l], pf)
            main.wait_stream(pf)

        for t in range(warmup):
            xbuf.copy_(xs[t:t + 1])
            enqueue()
        torch.cuda.synchronize()
        g_ = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_):
            enqueue()
        torch.cuda.synchronize()
        recs, pfr, routed = [], [], []
        t0 = time.perf_counter()
        for t in range(warmup, warmup + steps):
            xbuf.copy_(xs[t:t + 1])
            g_.replay()
            recs.append(torch.stack([L.miss_rec[:4] for L in layers]))
            pfr.append(torch.stack([pr[:nw] for pr in precs]))
            routed.append(idx[:, 0, :].clone())
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        r = torch.stack(recs).cpu().numpy()
        q = torch.stack(pfr).cpu().numpy()
        ro = torch.stack(routed).cpu().numpy()
        assert (r[:, :, 0] == 0).all() and (q[:, :, 0] == 0).all(), "cache capacity error"
        fetched = used = 0
        for t in range(steps - 1):
            for l in range(n_layers):
                n = int(q[t, l, 1])
                got = set(int(e) for e in q[t, l, 5:5 + n])
                fetched += n
                used += len(got & set(int(e) for e in ro[t + 1, l]))
        misses, pref = float(r[:, :, 1].sum()), float(q[:, :, 1].sum())
        runs.append({"m": m, "tokens_per_s": round(steps / dt, 2),
                     "hit_rate": round(float(r[:, :, 3].sum()) / (steps * n_layers * k), 4),
                     "routed_misses_per_token": round(misses / steps, 2),
                     "prefetched_per_token": round(pref / steps, 2),
                     "blobs_over_pcie_per_token": round((misses + pref) / steps, 2),
                     "prefetch_accuracy": round(used / max(fetched, 1), 4),
                     "h2d_GBps": round((misses + pref) * eb / dt / 1e9, 2)})
        del layers, bufs
        torch.cuda.empty_cache()
    return {"workload": f"cache35b: {n_layers} layers, {S} VRAM slots per layer, batch 1; runner-up prefetch",
            "executor": "moe_cached_layer_enqueue_prefetch x 40 layers in one HIP graph (prefetch stream joined "
                        "at the end of the step)",
            "warmup_steps": warmup, "timed_steps": steps, "runs": runs}


def cache_split_leg(fmt, hosts, routers, stride, warmup, steps, threads):
    """The decode scheduler's split of each step's misses between GPU cache fills
    and host CPU experts (moe_cached_layer_forward_split, host-waiting executor):
    PCIe H2D bandwidth (one layer's pinned host pool copied to the device) and the
    host expert kernel's blob bandwidth (moe_host_expert_ffn on 32 blobs of the
    pinned pool) are measured first; q* = B_host / (B_host + B_pcie) is the share
    that keeps both sides equally busy.  Then the 40-layer cache workload runs at
    q = 0, q* and 0.5."""
    import numpy as np
    import torch

    from block_scaled_fp4_gemv_amd import binding as B
    from block_scaled_fp4_gemv_amd import synth as sy

    wl = sy.WORKLOADS["cache35b"]
    H, E, F, k, S = wl.H, wl.E, wl.F, wl.k, wl.slots
    n_layers = len(hosts)
    eb = B.moe_expert_bytes(fmt, H, F)
    # PCIe H2D: one layer's pool
    dev = torch.empty_like(hosts[0], device="cuda")
    dev.copy_(hosts[0], non_blocking=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        dev.copy_(hosts[0], non_blocking=True)
    torch.cuda.synchronize()
    b_pcie = 3 * hosts[0].numel() / (time.perf_counter() - t0)
    del dev
    # host expert kernel on blobs of the pinned pool
    hp = hosts[0].numpy()
    blobs = [hp[e * stride:e * stride + eb] for e in range(32)]
    xh = sy.ar1_sequence(0, wl.cfg_id, 1, H)[0]
    B.moe_host_expert_ffn(fmt, H, F, blobs, [xh] * 32, threads=threads)
    t0 = time.perf_counter()
    for _ in range(5):
        B.moe_host_expert_ffn(fmt, H, F, blobs, [xh] * 32, threads=threads)
    b_host = 5 * 32 * eb / (time.perf_counter() - t0)
    q_star = b_host / (b_host + b_pcie)
    xs = torch.from_numpy(sy.ar1_sequence(0, wl.cfg_id, warmup + steps, H)).cuda()
    ws = torch.empty(B.moe_cached_layer_workspace(fmt, 1, H, F, k, E) + 256, dtype=torch.uint8, device="cuda")
    hws = B.new_split_host_workspace(1, H, F, k)
    bufs = [torch.empty(s_, dtype=d, device="cuda") for s_, d in
            (((1, k), torch.int32), ((1, k), torch.float32), (k, torch.int32), (k, torch.int32), ((1, H), torch.uint16))]
    copy = torch.cuda.Stream()
    runs = []
    for q in (0.0, round(q_star, 3), 0.5):
        layers = [B.CachedLayer(routers[l], hosts[l], torch.zeros(S * stride, dtype=torch.uint8, device="cuda"),
                                E, S, 1, k) for l in range(n_layers)]
        defers = [torch.cuda.Event() for _ in range(n_layers)]
        tot = np.zeros(3, np.int64)
        for t in range(warmup + steps):
            if t == warmup:
                torch.cuda.synchronize()
                tot[:] = 0
                t0 = time.perf_counter()
            x = xs[t:t + 1]
            for l, L in enumerate(layers):
                tot += B.moe_cached_layer_forward_split(fmt, stride, H, F, E, k, L, x, *bufs, ws, q, hws, defers[l],
                                                        threads=threads, copy_stream=copy)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        runs.append({"q": q, "tokens_per_s": round(steps / dt, 2),
                     "hit_rate": round(float(tot[0]) / (steps * n_layers * k), 4),
                     "misses_per_token": round(float(tot[1]) / steps, 2),
                     "cpu_served_per_token": round(float(tot[2]) / steps, 2)})
        del layers
        torch.cuda.empty_cache()
    return {"workload": f"cache35b: {n_layers} layers, {S} VRAM slots per layer, batch 1; misses split between "
                        f"GPU fills and host CPU experts",
            "executor": "moe_cached_layer_forward_split per layer (host waits on each layer's miss record)",
            "pcie_h2d_GBps": round(b_pcie / 1e9, 2), "host_expert_GBps": round(b_host / 1e9, 2),
            "host_threads": threads, "q_star": round(q_star, 3),
            "warmup_steps": warmup, "timed_steps": steps, "runs": runs}


class DecodeStack:
    """Batch-1 decode through a stack of resident layers, one moe_layer_forward
    per layer (each layer's down kernel reading the next layer's router ahead),
    the whole step captured in one HIP graph."""

    def __init__(self, fmt, wl, pools, routers, stride, n_layers, xs, read_ahead=True):
        import torch

        from block_scaled_fp4_gemv_amd import binding as B

        H, E, F, k = wl.H, wl.E, wl.F, wl.k
        self.n_layers, self.n_states = n_layers, xs.shape[0]
        self.xs_dev = torch.from_numpy(xs).cuda()
        self.x = torch.empty((1, H), dtype=torch.uint16, device="cuda")
        self.idx = [torch.empty((1, k), dtype=torch.int32, device="cuda") for _ in range(n_layers)]
        w = [torch.empty((1, k), dtype=torch.float32, device="cuda") for _ in range(n_layers)]
        out = [torch.empty((1, H), dtype=torch.uint16, device="cuda") for _ in range(n_layers)]
        lws = [B.new_layer_workspace(fmt, 1, H, F, k, E) for _ in range(n_layers)]

        def step():
            for l in range(n_layers):
                B.moe_layer_forward(fmt, pools[l], stride, H, F, E, k, self.x, routers[l], topk_idx=self.idx[l],
                                    topk_w=w[l], out=out[l], ws=lws[l],
                                    warm=routers[(l + 1) % n_layers] if read_ahead else None)

        # eager warm-up, then capture one step in a HIP graph
        self.x.copy_(self.xs_dev[0:1])
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        self.g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g):
            step()
        torch.cuda.synchronize()
        # the graph's buffers: each layer's routing and output of the last replay
        self.topk_w, self.out, self.ws = w, out, lws

    def replay(self, i):
        j = i % self.n_states
        self.x.copy_(self.xs_dev[j:j + 1])
        self.g.replay()

    def time(self, warmup, steps):
        """ms per step over `steps` timed replays (HIP events) after `warmup`."""
        import torch
        for i in range(warmup):
            self.replay(i)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for i in range(steps):
            self.replay(warmup + i)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps

    def routing_persistence(self, start, n):
        """How well the previous step's routing of the same layer predicts this
        step's (the predictor of a speculative weight stream): over n more
        steps, the share of each layer's k routed experts that the layer also
        routed at the previous step, and the share routed at the same rank."""
        import numpy as np
        import torch
        if n < 2:
            return None
        prev, in_set, same_rank, tot = None, 0, 0, 0
        for i in range(n):
            self.replay(start + i)
            cur = torch.stack(self.idx).cpu().numpy().reshape(self.n_layers, -1)
            if prev is not None:
                for l in range(self.n_layers):
                    in_set += len(set(cur[l].tolist()) & set(prev[l].tolist()))
                    same_rank += int(np.sum(cur[l] == prev[l]))
                    tot += cur.shape[1]
            prev = cur
        return {"prev_step_set_overlap": round(in_set / tot, 4), "prev_step_same_rank": round(same_rank / tot, 4),
                "steps": n, "layers": self.n_layers}


def oracle_sample(fmt, wl, x, routers, batch, what):
    """The oracle as it stands (NumPy fp64, dequant included) on a bounded sample:
    x's rows through one layer per router, every layer with the experts of
    `batch` (generated outside the timed region).  Returns tokens/s and the sample."""
    import numpy as np

    from block_scaled_fp4_gemv_amd import synth as sy
    from oracle import moe

    class View:
        def __getitem__(self, e):
            return sy.expert_view(batch, int(e))

    ex = View()
    t0 = time.perf_counter()
    for R in routers:
        moe.moe_layer(fmt, x, np.asarray(R), ex, wl.k)
    dt = time.perf_counter() - t0
    return {"tokens_per_s": round(x.shape[0] / dt, 4), "kind": "oracle", "cores": os.cpu_count(),
            "sample": f"{what}: {x.shape[0]} token(s) through {len(routers)} layer(s) "
                      f"(NumPy fp64 oracle incl. dequant; {dt:.1f} s)"}


def c4_leg(args):
    """The 753B-class stack (hidden 6144, 256 experts, top-8, width 2048, NVFP4):
    batch-1 decode through its 8 layers (layer 0's experts generated once, every
    other layer its own device copy) and the 4096-token prefill of one layer."""
    import torch

    from block_scaled_fp4_gemv_amd import synth as sy

    wl = sy.WORKLOADS["decode753b"]
    fmt = 1
    batch0 = [] if args.c4_cpu and not args.no_cpu_baseline else None
    pools, routers, stride, _ = build_stack(wl, fmt, wl.layers, args.threads, replicate=True, batch0=batch0)
    xs = sy.ar1_sequence(0, wl.cfg_id, wl.steps, wl.H)
    dec = DecodeStack(fmt, wl, pools, routers, stride, wl.layers, xs)
    ms = dec.time(args.warmup, args.c4_steps)
    layer_us = ms * 1000.0 / wl.layers
    nb = algorithmic_bytes(wl, fmt)
    gbps = nb["layer_total"] / (layer_us * 1e-6) / 1e9
    res = {"decode": {"workload": f"decode753b: {wl.layers} stacked MoE layers, hidden {wl.H}, {wl.E} experts, "
                                  f"top-{wl.k}, expert width {wl.F}, nvfp4, batch 1 (layer 0's experts replicated "
                                  f"to every layer's own device pool)",
                      "tokens_per_s": round(1000.0 / ms, 2), "layer_us": round(layer_us, 3),
                      "bytes_per_layer": nb["layer_total"], "hbm_GBps": round(gbps, 1),
                      "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4), "steps": args.c4_steps,
                      "timing": "one HIP graph per token, HIP events over the timed replays"}}
    log(f"C4 decode: {res['decode']}")
    routers_host = [r.cpu().numpy() for r in routers]
    del dec, pools, routers
    torch.cuda.empty_cache()
    if args.c4_prefill_reps > 0:
        res["prefill"] = prefill_leg("prefill753b", fmt, args.c4_prefill_reps, args.threads)
        log(f"C4 prefill: {res['prefill']['layer_us']} us/layer")
        torch.cuda.empty_cache()
    if batch0:
        # the replicated stack's layers all carry layer 0's experts, which are also
        # the first weight set of the 4096-token prefill
        res["decode"]["cpu_oracle"] = oracle_sample(fmt, wl, xs[:1], routers_host, batch0[0],
                                                    "decode753b, first decode token")
        pw = sy.WORKLOADS["prefill753b"]
        xp = sy.token_rows(0, pw.cfg_id, args.c4_cpu, pw.H)
        if "prefill" in res:
            res["prefill"]["cpu_oracle"] = oracle_sample(fmt, pw, xp, [sy.router(0, pw.wcfg, 0, pw.E, pw.H)],
                                                         batch0[0], "prefill753b, first tokens of the input")
        log(f"C4 oracle: decode {res['decode']['cpu_oracle']}")
    return res


def algorithmic_bytes(wl, fmt):
    """Bytes one decode token must move, per layer: weights of the k routed experts
    (codes + block scales + tensor scales), the fp32 router, and the activations."""
    from block_scaled_fp4_gemv_amd import binding as B
    eb = B.moe_expert_bytes(fmt, wl.H, wl.F) - 256 + (12 if fmt == 1 else 0)
    router = wl.E * wl.H * 4
    act_route = wl.H * 2 + wl.k * 8
    act_ffn = wl.H * 2 + wl.k * wl.F * 2 * 2 + wl.H * 2 + wl.k * 8
    return dict(expert=wl.k * eb, router=router, ffn_total=wl.k * eb + act_ffn,
                route_total=router + act_route, layer_total=wl.k * eb + router + act_route + act_ffn)


MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}
MX_NATIVE_INSTR = ("v_mfma_scale_f32_16x16x128_f8f6f4, FP4 weights x FP8 activations (two terms per bf16 value, "
                   "so the expert flops count twice in the instruction's own rate)")


def prefill_leg(name, fmt_override, reps, threads, mx_native=False, prepared_router=True, cpu_tokens=0):
    """Time moe_layer_forward over a T-token prefill of one layer (grouped MFMA path)."""
    import numpy as np
    import torch

    from block_scaled_fp4_gemv_amd import binding as B
    from block_scaled_fp4_gemv_amd import synth as sy

    wl = sy.WORKLOADS[name]
    fmt = fmt_override or wl.fmt
    H, E, F, k, T = wl.H, wl.E, wl.F, wl.k, wl.T
    sy.set_threads(threads)
    stride = B.blob_stride(fmt, H, F)
    # two layers used alternately, so that more than twice the 256 MB MALL is
    # touched between reuses of a weight set
    pools, Rs = [], []
    batch0 = None
    for l in range(2):
        host = np.empty(E * stride, np.uint8)
        batch = sy.experts(fmt, 0, wl.wcfg, l, 0, E, H, F, wl.w_std)
        B.pack_layer(fmt, H, F, batch, host, stride, threads=threads)
        if l == 0 and cpu_tokens > 0:
            batch0 = batch
        del batch
        pools.append(torch.from_numpy(host).cuda())
        R = torch.from_numpy(sy.router(0, wl.wcfg, l, E, H)).cuda()
        # the router's bf16 split is made once per weight set, not per call
        Rs.append(B.PreparedRouter(R) if prepared_router else R)
        del host, R
    x = torch.from_numpy(sy.token_rows(0, wl.cfg_id, T, H)).cuda()
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H), dtype=torch.uint16, device="cuda")
    ws = B.new_layer_workspace(fmt, T, H, F, k, E)
    rep = [0]

    def run():
        l = rep[0] % 2
        rep[0] += 1
        B.moe_layer_forward(fmt, pools[l], stride, H, F, E, k, x, Rs[l], topk_idx=idx, topk_w=w, out=out, ws=ws,
                            flags=B.MOE_LAYER_MX_NATIVE if mx_native else 0)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    # one HIP graph per weight set (the layer's kernels replayed without host
    # launch gaps, as in the decode step)
    graphs = []
    for l in range(2):
        g = torch.cuda.CUDAGraph()
        rep[0] = l
        with torch.cuda.graph(g):
            run()
        graphs.append(g)
    torch.cuda.synchronize()
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        graphs[i % 2].replay()
        b.record()
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(b) for a, b in evs])) * 1000
    used = int(torch.unique(idx).numel())
    eb = B.moe_expert_bytes(fmt, H, F) - 256 + (12 if fmt == 1 else 0)
    bytes_alg = used * eb + E * H * 4 + T * H * 2 * 2 + T * k * 8
    flops_mfma = 2.0 * T * k * (2 * F * H + H * F)
    flops_router = 2.0 * T * E * H
    t = us * 1e-6
    native = fmt == 2 and mx_native
    hbm_frac = bytes_alg / t / (HBM_PEAK_GBPS * 1e9)
    mf = flops_mfma / t / 1e12
    fmt_name = {1: "nvfp4", 2: "mxfp4", 3: "fp8"}[fmt]
    cpu = None
    if batch0 is not None:
        del pools, graphs
        cpu = oracle_sample(fmt, wl, x[:cpu_tokens].cpu().numpy(), [sy.router(0, wl.wcfg, 0, E, H)], batch0,
                            f"{name}, first tokens of the input")
    return {**({"cpu_oracle": cpu} if cpu else {}),
            "workload": f"{name}: {T} tokens through one layer, hidden {H}, {E} experts, top-{k}, "
                        f"width {F}, {fmt_name}",
            "tokens_per_s": round(T / t, 1), "layer_us": round(us, 2), "experts_used": used,
            "algorithmic_bytes": bytes_alg, "hbm_GBps": round(bytes_alg / t / 1e9, 1),
            "hbm_frac": round(hbm_frac, 4), "expert_mfma_tflops": round(mf, 2),
            "mfma_instruction": (MX_NATIVE_INSTR if native else
                                 "v_mfma_f32_16x16x32_bf16 (weights dequantized in registers)"),
            "mfma_util_vs_bf16_peak": round(mf / MFMA_PEAK_TFLOPS["bf16"], 4),
            **({"mfma_util_vs_fp8_peak": round(mf / MFMA_PEAK_TFLOPS["fp8"], 4)} if native else {}),
            "mfma_util_vs_fp4_peak": round(mf / MFMA_PEAK_TFLOPS["fp4"], 4),
            "roofline_frac": round(max(hbm_frac, flops_mfma / (MFMA_PEAK_TFLOPS["bf16"] * 1e12) / t), 4),
            "router_fp32_gflop": round(flops_router / 1e9, 2),
            "timing": f"moe_layer_forward captured in one HIP graph per weight set (two sets, replayed "
                      f"alternately); HIP events around each replay, median of {reps}",
            "router": ("prepared once per weight set (moe_router_prepare: fp32 router + its bf16 split)"
                       if prepared_router else "plain fp32 router (split into bf16 planes on every call)"),
            **({"role": f"compute-bound point: {T * k // E} rows per expert on average, "
                        f"{flops_mfma / bytes_alg:.0f} flop per algorithmic byte"} if name == "prefill35b_16k" else {})}


def prefill_stream_leg(fmt, hosts, pools, routers, stride, reps):
    """Prefill with the experts in pinned host memory (moe_prefill_streamed): the
    2048-token prefill35b input through every layer of the stack, each layer's E
    blobs copied over PCIe into one of two VRAM pools while the previous layer
    computes.  Also timed alone: the same copies without compute, and the same
    layers computed from resident pools (pools)."""
    import numpy as np
    import torch

    from block_scaled_fp4_gemv_amd import binding as B
    from block_scaled_fp4_gemv_amd import synth as sy

    wl = sy.WORKLOADS["prefill35b"]
    H, E, F, k, T = wl.H, wl.E, wl.F, wl.k, wl.T
    L = len(hosts)
    x = torch.from_numpy(sy.token_rows(0, wl.cfg_id, T, H)).cuda()
    outs = [torch.empty((T, H), dtype=torch.uint16, device="cuda") for _ in range(L)]
    idx = torch.empty((L, T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((L, T, k), dtype=torch.float32, device="cuda")
    ps = B.PrefillStream(E, stride)
    ws = torch.empty(B.moe_prefill_streamed_workspace(fmt, T, H, F, k, E), dtype=torch.uint8, device="cuda")
    main = torch.cuda.current_stream()

    def streamed():
        B.moe_prefill_streamed(fmt, stride, H, F, E, k, hosts, routers, x, outs, idx, w, ps, ws)

    def compute_only():
        for l in range(L):
            B.moe_layer_forward(fmt, pools[l], stride, H, F, E, k, x, routers[l], topk_idx=idx[l], topk_w=w[l],
                                out=outs[l], ws=ws)

    def copy_only():
        for l in range(L):
            ps.pools[l % 2].copy_(hosts[l], non_blocking=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(main)
            fn()
            b.record(main)
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        return float(np.median(ms))

    t_stream = timed(streamed)
    t_copy = timed(copy_only)
    t_comp = timed(compute_only)
    nbytes = L * E * stride
    hidden = (t_copy + t_comp - t_stream) / t_comp if t_comp > 0 else 0.0
    fmt_name = {1: "nvfp4", 2: "mxfp4", 3: "fp8"}[fmt]
    return {"workload": f"prefill35b input ({T} tokens) through {L} layers of the decode35b stack, {fmt_name}, "
                        f"every layer's {E} experts streamed from pinned host memory",
            "executor": "moe_prefill_streamed (two VRAM pools, copy stream + events)",
            "ms_per_prefill": round(t_stream, 3), "tokens_per_s": round(T / (t_stream * 1e-3), 1),
            "h2d_bytes": nbytes, "h2d_GBps": round(nbytes / (t_stream * 1e-3) / 1e9, 2),
            "copy_only_ms": round(t_copy, 3), "copy_only_GBps": round(nbytes / (t_copy * 1e-3) / 1e9, 2),
            "compute_only_ms": round(t_comp, 3),
            "compute_hidden_frac": round(min(1.0, max(0.0, hidden)), 4),
            "timing": f"HIP events on the compute stream, median of {reps} passes after one warm-up pass"}


def measured_traffic(n_layers_run, n_layers_default):
    """HBM bytes per decode layer from the committed request-size counter runs, if the
    kernel sources are unchanged since they were taken (else None)."""
    import glob
    import hashlib
    path = os.path.join(ROOT, "profiles", "decode35b_traffic.json")
    if not os.path.exists(path) or n_layers_run != n_layers_default:
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "block_scaled_fp4_gemv_amd", "csrc", "*"))):
        h.update(open(f, "rb").read())
    if h.hexdigest() != rec.get("sources_sha256"):
        return None
    return int(rec["decode_layer_read_bytes"] + rec["decode_layer_write_bytes"])


def cpu_baseline(wl, fmt, xs, n_steps, n_layers):
    """The oracle as it stands, on the first n_steps tokens of the same stack."""
    import numpy as np

    from block_scaled_fp4_gemv_amd import synth as sy
    from oracle import moe

    try:
        from threadpoolctl import threadpool_info
        pools = threadpool_info()
        blas_threads = max([d.get("num_threads", 1) for d in pools] + [1])
        blas = ", ".join(f"{d.get('internal_api')} {d.get('version')} ({d.get('num_threads')} threads)"
                         for d in pools if d.get("user_api") == "blas") or "none found"
    except Exception:  # pragma: no cover
        blas_threads, blas = 1, "unknown"
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu_model)
    except OSError:  # pragma: no cover
        pass

    class Lazy:
        def __init__(self, l):
            self.l, self.c = l, {}

        def __getitem__(self, e):
            if e not in self.c:
                b = sy.experts(fmt, 0, wl.wcfg, self.l, e, 1, wl.H, wl.F, wl.w_std)
                self.c[e] = sy.expert_view(b, 0)
            return self.c[e]

    layers = [(sy.router(0, wl.wcfg, l, wl.E, wl.H), Lazy(l)) for l in range(n_layers)]
    # weights are generated outside the timed region (the GPU leg also starts resident)
    for t in range(n_steps):
        for R, ex in layers:
            idx, _, _ = moe.route(xs[t:t + 1], R, wl.k)
            for e in idx.ravel():
                ex[int(e)]
    t0 = time.perf_counter()
    for t in range(n_steps):
        for R, ex in layers:
            moe.moe_layer(fmt, xs[t:t + 1], R, ex, wl.k)
    dt = time.perf_counter() - t0
    return dict(value=n_steps / dt, unit="tok/s", cores=int(blas_threads), kind="oracle",
                sample=f"first {n_steps} decode tokens through all {n_layers} layers "
                       f"(NumPy fp64 oracle incl. dequant; {dt:.1f} s)",
                host_cpus=os.cpu_count(), cpu_model=cpu_model, blas=blas)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from block_scaled_fp4_gemv_amd import binding as B
    from block_scaled_fp4_gemv_amd import synth as sy

    wl = sy.WORKLOADS[args.workload]
    fmt = args.fmt or wl.fmt
    n_layers = args.layers or wl.layers
    B.lib()
    torch.cuda.init()
    log(f"workload {wl.name}: {n_layers} layers H={wl.H} E={wl.E} k={wl.k} F={wl.F} fmt={fmt}")
    want_cache = args.cache != "none" and wl.name == "decode35b"
    pools, routers, stride, hosts = build_stack(wl, fmt, n_layers, args.threads, keep_host=want_cache,
                                                replicate=args.replicate_layers)
    H, E, F, k = wl.H, wl.E, wl.F, wl.k

    n_states = wl.steps
    xs = sy.ar1_sequence(0, wl.cfg_id, n_states, H)
    dec = DecodeStack(fmt, wl, pools, routers, stride, n_layers, xs, read_ahead=not args.no_read_ahead)
    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ms_step = dec.time(args.warmup, args.steps)
    tok_s = 1000.0 / ms_step
    log(f"timed {args.steps} steps: {ms_step * 1000:.1f} us/step, {tok_s:.1f} tok/s")
    persistence = dec.routing_persistence(args.warmup + args.steps, args.persistence_steps)
    log(f"routing persistence: {persistence}")

    # one layer launch = the layer's kernels inside the timed graph replays: its
    # mean duration is the timed region (HIP events) divided by steps x layers
    layer_us = ms_step * 1000.0 / n_layers

    nb = algorithmic_bytes(wl, fmt)
    layer_gbps = nb["layer_total"] / (layer_us * 1e-6) / 1e9
    stack_bytes = nb["layer_total"] * n_layers
    stream_gbps = stack_bytes * tok_s / 1e9

    res = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {1: "nvfp4 weights, bf16 activations, fp32 accumulate",
                  2: "mxfp4 weights, bf16 activations, fp32 accumulate",
                  3: "fp8-e4m3 weights, bf16 activations, fp32 accumulate"}[fmt],
        "data": (f"synthetic (seeded N(0,{wl.w_std}) weights quantized to the block format; AR(1) bf16 states"
                 + ("; layer 0's experts replicated to every layer's own device pool" if args.replicate_layers
                    else "") + ")"),
        "config": {"workload": f"{wl.name}: {n_layers} stacked MoE layers, hidden {H}, {E} experts, "
                               f"top-{k}, expert width {F}, batch 1",
                   "layers": n_layers, "hidden": H, "experts": E, "top_k": k, "expert_width": F,
                   "format": {1: "nvfp4", 2: "mxfp4", 3: "fp8"}[fmt], "batch": 1,
                   "graph": "one HIP graph per step",
                   "read_ahead": None if args.no_read_ahead else
                   "each layer's down kernel warms the next layer's router (moe_layer_forward_prefetch)"},
        "weight_stream_GBps": round(stream_gbps, 1),
        "routing_persistence": persistence,
        "weight_stream_frac_of_hbm": round(stream_gbps / HBM_PEAK_GBPS, 4),
        "roofline": {"kernel": "moe_layer_forward decode layer (router GEMV, gate/up+SwiGLU with "
                               "in-block top-k, down+combine: 3 kernels)",
                     "bound": "hbm", "achieved": round(layer_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(layer_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": (measured_traffic(n_layers, wl.layers)
                                 if wl.name == "decode35b" and fmt == 1 else None),
                     "bytes_per_launch": nb["layer_total"], "avg_launch_us": round(layer_us, 3),
                     "launch_timing": "timed graph replays / (steps x layers), HIP events"},
    }
    if want_cache:
        log(f"cache leg {args.cache} ...")
        res["cache"] = cache_leg(args.cache, fmt, hosts, routers, stride, args.cache_warmup, args.cache_steps,
                                 host_sync=args.cache_host_sync, elastic_steps=args.cache_elastic_steps)
        log(f"cache: {res['cache']['tokens_per_s']} tok/s, hit rate {res['cache']['hit_rate']}, "
            f"{res['cache']['h2d_GBps']} GB/s H2D")
        if args.cache_split_steps > 0:
            log("cache split leg ...")
            res["cache_split"] = cache_split_leg(fmt, hosts, routers, stride, args.cache_split_warmup,
                                                 args.cache_split_steps, args.threads)
            log(f"cache split: {res['cache_split']}")
        if args.cache_prefetch_steps > 0:
            log("cache prefetch leg ...")
            res["cache_prefetch"] = cache_prefetch_leg(fmt, hosts, routers, stride, args.cache_warmup,
                                                       args.cache_prefetch_steps)
            log(f"cache prefetch: {res['cache_prefetch']['runs']}")
        if args.cache_shared_steps > 0:
            log("shared-cache leg ...")
            res["cache_shared"] = cache_shared_leg(fmt, hosts, stride, args.cache_warmup, args.cache_shared_steps)
            log(f"shared cache: per-layer {res['cache_shared']['per_layer']}, shared {res['cache_shared']['shared']}")
        if args.prefill_stream_reps > 0:
            log("streamed-prefill leg ...")
            res["prefill_stream"] = prefill_stream_leg(fmt, hosts, pools, routers, stride, args.prefill_stream_reps)
            log(f"streamed prefill: {res['prefill_stream']['ms_per_prefill']} ms per prefill, "
                f"{res['prefill_stream']['h2d_GBps']} GB/s H2D, compute hidden "
                f"{res['prefill_stream']['compute_hidden_frac']}")
        del hosts
    if args.prefill != "none":
        log(f"prefill leg {args.prefill} ...")
        del pools, dec
        torch.cuda.empty_cache()
        res["prefill"] = prefill_leg(args.prefill, args.fmt, args.prefill_reps, args.threads, args.mx_native,
                                     prepared_router=not args.plain_router,
                                     cpu_tokens=0 if args.no_cpu_baseline else args.cpu_prefill_tokens)
        log(f"prefill: {res['prefill']['layer_us']} us/layer, {res['prefill']['tokens_per_s']} tok/s")
        if args.prefill == "prefill35b" and args.compute_bound_reps > 0:
            log("compute-bound prefill point prefill35b_16k ...")
            torch.cuda.empty_cache()
            res["prefill_compute_bound"] = prefill_leg("prefill35b_16k", args.fmt, args.compute_bound_reps,
                                                       args.threads, args.mx_native,
                                                       prepared_router=not args.plain_router)
            log(f"prefill35b_16k: {res['prefill_compute_bound']['layer_us']} us/layer, bf16 MFMA "
                f"{res['prefill_compute_bound']['mfma_util_vs_bf16_peak']}")
    if args.c4_steps > 0 and wl.name == "decode35b":
        log("753B-class leg ...")
        torch.cuda.empty_cache()
        res["c4"] = c4_leg(args)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline(wl, fmt, xs, args.cpu_sample_steps, n_layers)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
