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


# ------------------------------------------------------------ elastic resize

def _last_use(trace):
    """Expert -> index of its last access in the flattened pair order (brute force)."""
    last, i = {}, 0
    for step in trace:
        for e in np.asarray(step).ravel():
            last[int(e)] = i
            i += 1
    return last


@pytest.mark.parametrize("seed,S,S_new", [(0, 8, 5), (1, 8, 3), (2, 8, 8), (3, 8, 12), (4, 12, 1),
                                          (5, 6, 9)])
def test_resize_stamp_and_list_forms_agree(seed, S, S_new):
    """Both formulations give the same slot table after a resize and at every
    later step; the kept experts are the S_new most recently used residents,
    found here by brute force from the raw access sequence."""
    rng = np.random.default_rng(seed)
    E = 24
    a, b = lru.StampLRU(E, S), lru.ListLRU(E, S)
    trace = [rng.integers(0, E, (2, 2)) for _ in range(40)]
    for st in trace:
        assert a.step(st)["status"] == lru.OK and b.step(st)["status"] == lru.OK
    resident = [int(e) for e in a.slot_expert if e >= 0]
    last = _last_use(trace)
    want = set(sorted(resident, key=lambda e: -last[e])[:S_new])
    before = a.slot_expert.copy()
    plan = a.resize(S_new)
    b.resize(S_new)
    assert a.S == S_new and np.array_equal(a.slot_expert, b.slot_table())
    assert set(int(e) for e in a.slot_expert if e >= 0) == want
    for t, e in enumerate(a.slot_expert):          # expert_slot is the inverse table
        if e >= 0:
            assert a.expert_slot[e] == t
    assert (a.expert_slot >= 0).sum() == len(want)
    for s_old, t in plan["all"]:                   # a kept expert below S_new never moves
        assert a.slot_expert[t] == before[s_old]
        assert (s_old == t) == (s_old < S_new)
    assert plan["in_place"] == [(s_old, t) for s_old, t in plan["all"] if s_old != t]
    for st in [rng.integers(0, E, (2, 2)) for _ in range(40)]:
        ra, rb = a.step(st), b.step(st)
        assert ra["status"] == rb["status"]
        if ra["status"] == lru.OK:
            assert np.array_equal(ra["pair_slot"], rb["pair_slot"])
        assert np.array_equal(a.slot_expert, b.slot_table())


def test_resize_grow_keeps_every_slot_and_adds_empty_ones():
    a = lru.StampLRU(16, 4)
    for e in (3, 7, 1, 9, 7):
        a.step(np.array([[e]]))
    before, stamps, clock = a.slot_expert.copy(), a.slot_stamp.copy(), a.clock
    plan = a.resize(7)
    assert list(a.slot_expert) == list(before) + [-1, -1, -1]
    assert list(a.slot_stamp) == list(stamps) + [0, 0, 0] and a.clock == clock
    assert plan["in_place"] == [] and plan["all"] == [(s, s) for s in range(4)]


def test_resize_shrink_fills_the_lowest_free_slots_in_old_slot_order():
    """Slots 0..5 hold experts 10..15, last used in the order 12, 15, 10, 14, 11, 13
    (13 most recent).  Shrinking to 3 keeps 13, 11, 14; 11 stays in slot 1; 13
    (old slot 3) and 14 (old slot 4) take the free slots 0 and 2 in ascending
    order of their old slot: 13 -> 0, 14 -> 2."""
    a = lru.StampLRU(16, 6)
    a.step(np.arange(10, 16).reshape(-1, 1))
    for e in (12, 15, 10, 14, 11, 13):
        a.step(np.array([[e]]))
    plan = a.resize(3)
    assert [int(e) for e in a.slot_expert] == [13, 11, 14]
    assert plan["in_place"] == [(3, 0), (4, 2)]
    assert plan["all"] == [(1, 1), (3, 0), (4, 2)]


def test_resize_working_set_hits_follow_the_capacity():
    """A cyclic working set of W = 6 experts: all hits while S >= W, none after
    shrinking to S = 5 (an LRU scan of S+1 items), all hits again one cycle after
    growing back to 6."""
    W = 6
    a = lru.StampLRU(32, 8)
    cycle = [np.array([[e]]) for e in range(W)]

    def run(n_cycles):
        hits = acc = 0
        for _ in range(n_cycles):
            for st in cycle:
                r = a.step(st)
                hits, acc = hits + r["n_hits"], acc + r["n_access"]
        return hits / acc

    run(1)
    assert run(3) == 1.0
    a.resize(5)
    assert run(3) == 0.0
    a.resize(W)
    run(1)
    assert run(3) == 1.0


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


# ------------------------------------------------ a cache shared by several layers

def _shared_trace(rng, n_layers, E, k, n_steps):
    """Per step, each layer's top-k accesses; layer j draws from a window of
    experts whose width grows with j (unequal demand)."""
    steps = []
    for t in range(n_steps):
        step = []
        for j in range(n_layers):
            width = k + 2 + 3 * j
            step.append(rng.choice(width, size=k, replace=False) + (t // 5) % (E - width + 1))
        steps.append(step)
    return steps


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_shared_cache_stamp_and_list_forms_agree(seed):
    """Layers taking turns on one keyed cache: the stamp form and the independent
    list form give the same slot table and the same records (in experts) at every
    layer step."""
    rng = np.random.default_rng(seed)
    n_layers, E, k, S = 4, 32, 3, 14
    st, li = lru.StampLRU(n_layers * E, S), lru.ListLRU(n_layers * E, S)
    vs = [lru.LayerView(st, j * E) for j in range(n_layers)]
    vl = [lru.LayerView(li, j * E) for j in range(n_layers)]
    for step in _shared_trace(rng, n_layers, E, k, 60):
        for j, acc in enumerate(step):
            a, b = vs[j].step(acc), vl[j].step(acc)
            assert a["status"] == b["status"] == lru.OK
            assert np.array_equal(a["pair_slot"], b["pair_slot"])
            assert np.array_equal(a["miss_expert"], b["miss_expert"]) and np.array_equal(a["miss_slot"], b["miss_slot"])
            assert np.all((a["miss_expert"] >= 0) & (a["miss_expert"] < E))
            assert np.array_equal(st.slot_expert, li.slot_table())


def test_shared_cache_holds_the_most_recent_keys():
    """Brute force from the raw access sequence: after every step the cache holds
    exactly the min(S, distinct) most recently used keys, whichever layer used them."""
    rng = np.random.default_rng(5)
    n_layers, E, k, S = 3, 24, 2, 9
    st = lru.StampLRU(n_layers * E, S)
    views = [lru.LayerView(st, j * E) for j in range(n_layers)]
    seq = []
    for step in _shared_trace(rng, n_layers, E, k, 80):
        for j, acc in enumerate(step):
            assert views[j].step(acc)["status"] == lru.OK
            seq += [j * E + int(e) for e in acc]
            last = {}
            for i, key in enumerate(seq):
                last[key] = i
            recent = sorted(last, key=lambda key: -last[key])[:S]
            assert set(int(v) for v in st.slot_expert if v >= 0) == set(recent)


def test_shared_cache_gives_a_busy_layer_the_idle_slots():
    """A worked case: layer 0 cycles through 6 experts, one per step, layer 1
    repeats one expert.  With 4 slots each, layer 0's cyclic scan of more experts
    than slots never hits; with the same 8 slots shared, the 7 keys in use fit and
    after the first cycle every access hits."""
    E = 16
    trace = [([t % 6], [9]) for t in range(30)]
    per = [lru.StampLRU(E, 4), lru.StampLRU(E, 4)]
    shared = lru.StampLRU(2 * E, 8)
    views = [lru.LayerView(shared, 0), lru.LayerView(shared, E)]
    miss_per = miss_shared = 0
    for t, (a0, a1) in enumerate(trace):
        for j, acc in enumerate((a0, a1)):
            rp, rs = per[j].step(acc), views[j].step(acc)
            if t >= 6:
                miss_per += rp["n_miss"]
                miss_shared += rs["n_miss"]
    assert miss_shared == 0
    assert miss_per == 24          # every layer-0 access of steps 6..29, none of layer 1


def test_shared_cache_with_one_layer_is_the_per_layer_cache():
    rng = np.random.default_rng(3)
    a, b = lru.StampLRU(40, 7), lru.StampLRU(40, 7)
    v = lru.LayerView(b, 0)
    for _ in range(50):
        acc = rng.choice(12, size=3, replace=False)
        ra, rb = a.step(acc), v.step(acc)
        assert np.array_equal(ra["pair_slot"], rb["pair_slot"]) and ra["n_miss"] == rb["n_miss"]


# ----------------------------------------------------------- predictive prefetch

def _ranked_trace(seed, n_steps, E, km):
    """Per step a ranked list of km distinct experts drifting slowly (the first k
    are routed, the rest runner-ups)."""
    rng = np.random.default_rng(seed)
    base = rng.permutation(E)
    out = []
    for t in range(n_steps):
        if t and rng.random() < 0.5:
            i, j = rng.integers(0, E, size=2)
            base[[i, j]] = base[[j, i]]
        out.append(base[:km].copy())
        rng.shuffle(base[:km + 3])
    return out


@pytest.mark.parametrize("seed", [0, 1])
def test_prefetch_stamp_and_list_forms_agree(seed):
    E, S, k, m = 40, 12, 4, 3
    st, li = lru.StampLRU(E, S), lru.ListLRU(E, S)
    for ranked in _ranked_trace(seed, 80, E, k + m):
        a, b = st.step(ranked[:k]), li.step(ranked[:k])
        assert np.array_equal(a["pair_slot"], b["pair_slot"])
        pa, pb = lru.prefetch_step(st, ranked), lru.prefetch_step(li, ranked)
        assert pa["status"] == pb["status"] == lru.OK
        assert np.array_equal(pa["miss_expert"], pb["miss_expert"]) and np.array_equal(pa["miss_slot"], pb["miss_slot"])
        assert np.array_equal(st.slot_expert, li.slot_table())


def test_prefetch_keeps_the_routed_experts_in_place():
    """The prefetch step never evicts or moves an expert the token was routed to,
    and afterwards every runner-up is resident."""
    E, S, k, m = 64, 14, 6, 4
    st = lru.StampLRU(E, S)
    for ranked in _ranked_trace(7, 60, E, k + m):
        r = st.step(ranked[:k])
        p = lru.prefetch_step(st, ranked)
        assert p["n_miss"] <= m
        assert np.array_equal(p["pair_slot"][:k], r["pair_slot"])
        assert all(st.expert_slot[e] >= 0 for e in ranked)


def test_prefetch_of_the_next_expert_removes_every_miss():
    """A worked case: a window of k experts slides by one each step (t .. t+k-1),
    and the runner-up is the next one (t+k).  Without prefetch every step after
    the first misses its newest expert; with it that expert was fetched one step
    earlier, so no routed access misses after the first step and every prefetch
    is used (prefetch accuracy 1)."""
    E, S, k, n = 50, 10, 4, 30
    plain, pre = lru.StampLRU(E, S), lru.StampLRU(E, S)
    miss_plain = miss_pre = used = fetched = 0
    prev_pf = set()
    for t in range(n):
        routed = list(range(t, t + k))
        rp = plain.step(routed)
        miss_plain += rp["n_miss"] if t else 0
        r = pre.step(routed)
        miss_pre += r["n_miss"] if t else 0
        used += len(prev_pf & set(routed))
        p = lru.prefetch_step(pre, routed + [t + k])
        prev_pf = set(int(e) for e in p["miss_expert"])
        fetched += len(prev_pf)
    assert miss_plain == n - 1 and miss_pre == 0
    assert fetched == n and used == n - 1

