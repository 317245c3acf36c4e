"""Pins for the oracle's LRU slot cache and the token-by-expert permutation."""
import numpy as np
import pytest

from oracle import lru, permute


def _compare_forms(trace, E, S):
    a, b = lru.StampLRU(E, S), lru.ListLRU(E, S)
    for step in trace:
        ra, rb = a.step(step), b.step(step)
        assert ra["status"] == rb["status"]
        if ra["status"] != lru.OK:
            continue
        assert np.array_equal(ra["pair_slot"], rb["pair_slot"])
        assert np.array_equal(ra["miss_expert"], rb["miss_expert"])
        assert np.array_equal(ra["miss_slot"], rb["miss_slot"])
        assert np.array_equal(a.slot_expert, b.slot_table())


@pytest.mark.parametrize("seed", range(6))
def test_stamp_and_list_forms_agree_random(seed):
    rng = np.random.default_rng(seed)
    E, S = 32, 8
    trace = []
    hot = rng.choice(E, 6, replace=False)
    for t in range(300):
        T, k = rng.integers(1, 3), rng.integers(1, 4)
        pool = hot if rng.random() < 0.6 else np.arange(E)
        trace.append(rng.choice(pool, (T, k)))     # duplicates within a step allowed
    _compare_forms(trace, E, S)


def test_stamp_and_list_forms_agree_top8_traces():
    rng = np.random.default_rng(9)
    E, S, k = 256, 64, 8
    prev = rng.choice(E, k, replace=False)
    trace = []
    for t in range(400):   # correlated steps: keep most of the previous top-8
        keep = prev[rng.random(k) < 0.8]
        fresh = rng.choice(np.setdiff1d(np.arange(E), keep), k - len(keep), replace=False)
        prev = np.concatenate([keep, fresh])
        trace.append(prev.copy())
    _compare_forms(trace, E, S)


def test_cyclic_scan_of_S_plus_1_never_hits():
    E, S = 20, 5
    steps = [[i % (S + 1)] for i in range(200)]
    assert lru.simulate_hit_rate(steps, E, S, skip=0) == 0.0


def test_fixed_set_within_capacity_always_hits_after_warmup():
    E, S = 50, 6
    rng = np.random.default_rng(1)
    steps = [list(rng.permutation([3, 7, 11, 40, 41, 49])[:4]) for _ in range(100)]
    first = lru.StampLRU(E, S)
    misses = sum(first.step(s)["n_miss"] for s in steps)
    assert misses == 6


def test_victim_order_empty_first_then_oldest():
    c = lru.StampLRU(10, 3)
    r = c.step([5]);      assert r["miss_slot"].tolist() == [0]
    r = c.step([6, 7]);   assert r["miss_slot"].tolist() == [1, 2]
    r = c.step([6]);      assert r["n_miss"] == 0
    r = c.step([8]);      assert r["miss_slot"].tolist() == [0]     # expert 5 is least recent
    r = c.step([9, 6]);   assert r["miss_slot"].tolist() == [2]     # 7 older than 8; 6 requested
    assert c.slot_expert.tolist() == [8, 6, 9]
    assert c.clock == 7 and c.slot_stamp.tolist() == [5, 7, 6]


def test_capacity_error_keeps_state():
    c = lru.StampLRU(10, 2)
    c.step([1, 2])
    before = c.state()
    r = c.step([3, 4, 1])
    assert r["status"] == lru.E_CAPACITY
    after = c.state()
    assert all(np.array_equal(x, y) for x, y in zip(before[:3], after[:3])) and before[3] == after[3]


def test_duplicates_within_step_and_pair_order():
    c = lru.StampLRU(16, 4)
    c.step([1, 2])
    r = c.step(np.array([[3, 1], [3, 2], [5, 3]]))
    assert r["n_miss"] == 2 and r["n_hits"] == 4 and r["n_access"] == 6
    assert r["n_hit_pairs"] == 2 and r["pair_order"].tolist() == [1, 3, 0, 2, 4, 5]
    assert r["miss_expert"].tolist() == [3, 5]


@pytest.mark.parametrize("T,k,E", [(16, 2, 8), (1, 8, 256), (300, 8, 64), (1, 1, 1)])
def test_permutation_properties(T, k, E):
    rng = np.random.default_rng(T)
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    perm, off = permute.permutation(idx, E)
    assert sorted(perm.tolist()) == list(range(T * k))
    assert np.array_equal(np.diff(off), np.bincount(idx.ravel(), minlength=E))
    flat = idx.ravel()
    for e in range(E):
        seg = perm[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)    # stable
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))      # library sort


def test_cache_policy_study_replays_the_oracle_lru():
    """The cache policy study (tests/cache_policy_study.py) replays the oracle LRU
    exactly when no policy is applied: prefetch m = 0, split q = 0 and a global
    pool of one layer all give the oracle's misses."""
    import cache_policy_study as ps
    from block_scaled_fp4_gemv_amd import synth as sy
    wl = sy.WORKLOADS["cache35b"]
    r = ps.rankings(24, n_layers=3)
    d = ps.simulate(r, wl.k, wl.slots, 0, warm=0)
    for layer in range(3):
        ref = lru.StampLRU(wl.E, wl.slots)
        for t in range(24):
            assert ref.step(r[layer, t, :wl.k])["n_miss"] == d["per_step_miss"][layer, t]
    assert d["prefetched_per_token"] == 0
    d4 = ps.simulate(r, wl.k, wl.slots, 4, warm=0)
    assert d4["prefetched_per_token"] > 0 and 0.0 <= d4["prefetch_accuracy"] <= 1.0
    g, c = ps.simulate_split(r, wl.k, wl.slots, 0.0, warm=0)
    assert c == 0 and g * 24 == d["per_step_miss"].sum()
    one = ps.simulate_global(r[:1], wl.k, wl.slots, warm=0)
    assert one * 24 == d["per_step_miss"][0].sum()
