"""Cache policies on the cache-constrained decode trace, evaluated on the CPU:
runner-up prefetch, a CPU / GPU miss split, and one LRU across all layers.

Prefetch:
For every layer of the cache35b stack (64 of 256 experts per layer in VRAM,
top-8, AR(1) decode states) the oracle's routing gives each step's expert
ranking.  The study replays the per-layer LRU of the cache (the oracle's
batch-aware rule: hits against the state at step start, victims among the
slots the step does not request, empty slots first, then the oldest stamp) and,
after each step, prefetches the experts ranked k+1 .. k+m that are not resident
(each into the least recently used slot that is neither requested nor just
prefetched, stamped as an access).  It reports, per token, the misses left on
the critical path, the prefetched blobs, the total blobs moved over PCIe and
the prefetch accuracy (share of prefetched experts that the same layer routes
to at the next step).  m = 0 is the plain predictor (a layer's top-k at step t
for step t+1), which names only resident experts and prefetches nothing.

Miss split: of a step's n misses the first round(q*n) are computed by the CPU
from the host pool and stay out of the cache (no slot, no stamp); the rest are
filled into the cache by the GPU.  It reports the GPU fills and the CPU expert
evaluations per token.

Global LRU: one pool of S*L slots shared by the L layers (keys (layer, expert),
the layers of a step looked up in order) against the per-layer pools.

    python tests/cache_policy_study.py [steps]
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from block_scaled_fp4_gemv_amd import synth as sy  # noqa: E402
from oracle import formats as fm  # noqa: E402


def rankings(steps, n_layers=None, depth=16):
    wl = sy.WORKLOADS["cache35b"]
    L = n_layers or wl.layers
    xs = fm.bf16_to_f64(sy.ar1_sequence(0, wl.cfg_id, steps, wl.H))
    out = np.empty((L, steps, depth), np.int64)
    for layer in range(L):
        z = xs @ sy.router(0, wl.wcfg, layer, wl.E, wl.H).astype(np.float64).T
        out[layer] = np.argsort(-z, axis=1, kind="stable")[:, :depth]
    return out


def simulate(ranks, k, S, m, warm):
    """Per-token averages over the steps after `warm` (all layers)."""
    L, steps, _ = ranks.shape
    crit = pf_loads = pf_used = pf_named = 0
    per_step_miss = np.zeros((L, steps), np.int64)
    for layer in range(L):
        slot_of, stamp, clock, prev = {}, {}, 0, set()
        for t in range(steps):
            top = [int(e) for e in ranks[layer, t, :k]]
            req = set(top)
            miss = []
            for e in top:
                if e not in slot_of and e not in miss:
                    miss.append(e)
            for e in miss:
                if len(slot_of) < S:
                    slot_of[e] = len(slot_of)
                else:
                    v = min((x for x in slot_of if x not in req), key=lambda x: stamp[x])
                    slot_of[e] = slot_of.pop(v)
                    stamp.pop(v)
            for e in top:
                clock += 1
                stamp[e] = clock
            per_step_miss[layer, t] = len(miss)
            if t >= warm:
                crit += len(miss)
                pf_used += len(prev & req)
            prev = set()
            for e in [int(x) for x in ranks[layer, t, k:k + m]]:
                if e in slot_of:
                    continue
                if len(slot_of) < S:
                    slot_of[e] = len(slot_of)
                else:
                    v = min((x for x in slot_of if x not in req and x not in prev), key=lambda x: stamp[x])
                    slot_of[e] = slot_of.pop(v)
                    stamp.pop(v)
                clock += 1
                stamp[e] = clock
                prev.add(e)
            if t >= warm:
                pf_loads += len(prev)
                pf_named += len(prev)
    n = steps - warm
    return dict(m=m, critical_misses_per_token=crit / n, prefetched_per_token=pf_loads / n,
                blobs_moved_per_token=(crit + pf_loads) / n, prefetch_accuracy=pf_used / max(pf_named, 1),
                per_step_miss=per_step_miss)


def simulate_split(ranks, k, S, q, warm):
    """(GPU fills, CPU expert evaluations) per token with the first round(q*n)
    misses of each step computed on the CPU and left out of the cache."""
    L, steps, _ = ranks.shape
    gpu = cpu = 0
    for layer in range(L):
        slot_of, stamp, clock = {}, {}, 0
        for t in range(steps):
            top = [int(e) for e in ranks[layer, t, :k]]
            req = set(top)
            miss = []
            for e in top:
                if e not in slot_of and e not in miss:
                    miss.append(e)
            n_cpu = int(np.floor(q * len(miss) + 0.5))
            for e in miss[n_cpu:]:
                if len(slot_of) < S:
                    slot_of[e] = len(slot_of)
                else:
                    v = min((x for x in slot_of if x not in req), key=lambda x: stamp[x])
                    slot_of[e] = slot_of.pop(v)
                    stamp.pop(v)
            for e in top:
                clock += 1
                if e in slot_of:
                    stamp[e] = clock
            if t >= warm:
                gpu += len(miss) - n_cpu
                cpu += n_cpu
    n = steps - warm
    return gpu / n, cpu / n


def simulate_global(ranks, k, total, warm):
    """Misses per token with one LRU of `total` slots over (layer, expert) keys."""
    L, steps, _ = ranks.shape
    slot_of, stamp, clock, misses = {}, {}, 0, 0
    for t in range(steps):
        for layer in range(L):
            top = [(layer, int(e)) for e in ranks[layer, t, :k]]
            req = set(top)
            miss = []
            for e in top:
                if e not in slot_of and e not in miss:
                    miss.append(e)
            for e in miss:
                if len(slot_of) < total:
                    slot_of[e] = len(slot_of)
                else:
                    v = min((x for x in slot_of if x not in req), key=lambda x: stamp[x])
                    slot_of[e] = slot_of.pop(v)
                    stamp.pop(v)
            for e in top:
                clock += 1
                stamp[e] = clock
            if t >= warm:
                misses += len(miss)
    return misses / (steps - warm)


def main():
    steps = int(sys.argv[1]) if len(sys.argv) > 1 else 192
    wl = sy.WORKLOADS["cache35b"]
    r = rankings(steps)
    for m in (0, 1, 2, 4, 8):
        d = simulate(r, wl.k, wl.slots, m, warm=64)
        d.pop("per_step_miss")
        print("prefetch", {kk: (round(v, 4) if isinstance(v, float) else v) for kk, v in d.items()})
    for q in (0.0, 0.25, 0.5, 0.75, 1.0):
        g, c = simulate_split(r, wl.k, wl.slots, q, warm=64)
        print(f"split q={q:.2f}: GPU fills {g:.2f} per token, CPU expert evaluations {c:.2f} per token")
    print(f"global LRU ({wl.slots * wl.layers} slots): "
          f"{simulate_global(r, wl.k, wl.slots * wl.layers, warm=64):.2f} misses per token")


if __name__ == "__main__":
    main()
