"""The device expert cache's policy ("Run Kimi 3.1 locally on one GPU",
sections "One GPU, three storage tiers" and "A drafter that leaves the answer
unchanged": with blocks wider than the cache LRU never hits, and a row-count
threshold for admission helps).  The reference in oracle/cache_policy.py is pinned to closed
forms first, then the library's policy (moe_cache_simulate, host code only,
no device call) must match it decision for decision on random traces."""
import numpy as np
import pytest

from oracle.cache_policy import CachePolicyRef


def _run_ref(n_layers, n_routed, n_cache, n_transient, admit, calls):
    p = CachePolicyRef(n_layers, n_routed, n_cache, n_transient, admit)
    return [p.plan(*c) for c in calls]


def _hits(res):
    return sum(sum(h) for _, h, _ in res)


# ----------------------------------------------------------------------------- pins of the reference
def test_ref_cyclic_scan_one_wider_than_lru_never_hits():
    # C slots, experts 0..C used one per call in a cycle: every access misses
    C = 6
    calls = [(0, [i % (C + 1)], [1]) for i in range(5 * (C + 1))]
    assert _hits(_run_ref(1, C + 1, C, 0, 0, calls)) == 0


def test_ref_working_set_that_fits_always_hits_after_first_use():
    C = 8
    ws = [1, 3, 4, 9]
    calls = [(0, ws, [1] * 4)] * 5
    res = _run_ref(1, 16, C, 0, 0, calls)
    assert [sum(h) for _, h, _ in res] == [0, 4, 4, 4, 4]


def test_ref_lru_victim_and_free_slots():
    # 2 cached slots: A, B fill slots 0, 1; C evicts the least recently used
    res = _run_ref(1, 10, 2, 0, 0, [(0, [1], [1]), (0, [2], [1]), (0, [1], [1]), (0, [3], [1]), (0, [2], [1])])
    slots = [s[0] for s, _, _ in res]
    hits = [h[0] for _, h, _ in res]
    assert slots == [0, 1, 0, 1, 0] and hits == [0, 0, 1, 0, 0]


def test_ref_layers_are_separate_keys():
    res = _run_ref(2, 4, 4, 0, 0, [(0, [1], [1]), (1, [1], [1]), (0, [1], [1]), (1, [1], [1])])
    assert [h[0] for _, h, _ in res] == [0, 0, 1, 1]


def test_ref_block_wider_than_cache_lru_zero_hits_admission_keeps_popular():
    # every block: 4 experts most rows use (ids 50..53) and 6 used by one row,
    # new ones each block (lower ids, so planned first).  A cache of 4: under
    # LRU the one-row experts take the cached slots every block and the
    # popular ones never stay (0 hits); keeping only experts with >= 3 rows
    # sends the one-row experts through transient slots and the popular
    # ones hit in every later block
    calls = []
    for b in range(5):
        rare = list(range(6 * b, 6 * b + 6))
        calls.append((0, rare + [50, 51, 52, 53], [1] * 6 + [9, 8, 5, 3]))
    lru = _run_ref(1, 64, 4, 8, 0, calls)
    adm = _run_ref(1, 64, 4, 8, 3, calls)
    assert _hits(lru) == 0
    assert [sum(h) for _, h, _ in adm] == [0, 4, 4, 4, 4]
    slot, hit, admitted = adm[1]
    assert all(s < 8 for s in slot[:6]) and admitted == [0] * 10


def test_ref_overflow_uses_transient_and_infeasible_raises():
    p = CachePolicyRef(1, 20, 2, 3, 0)
    slot, hit, adm = p.plan(0, [0, 1, 2, 3, 4], [1] * 5)
    assert sorted(slot) == [0, 1, 2, 3, 4] and adm == [1, 1, 0, 0, 0]
    with pytest.raises(ValueError):
        p.plan(0, list(range(6)), [1] * 6)


# ----------------------------------------------------------------------------- library == reference
def _trace(seed, n_layers, n_routed, n_calls, max_n, hot):
    g = np.random.default_rng(seed)
    calls = []
    for _ in range(n_calls):
        n = int(g.integers(1, max_n + 1))
        # a popular head and a uniform tail, like a skewed router
        pool = np.concatenate([np.arange(hot), g.permutation(n_routed)])
        ex = []
        for e in pool[g.permutation(len(pool))] if g.random() < 0.5 else pool:
            if e not in ex:
                ex.append(int(e))
            if len(ex) == n:
                break
        ex.sort()
        rows = [int(r) for r in g.integers(1, 17, size=len(ex))]
        calls.append((int(g.integers(0, n_layers)), ex, rows))
    return calls


@pytest.mark.parametrize("seed", range(12))
def test_library_policy_matches_reference(seed):
    import router_top_bucket_amd as moe
    g = np.random.default_rng(100 + seed)
    n_layers, n_routed = int(g.integers(1, 4)), int(g.integers(8, 60))
    max_n = min(n_routed, int(g.integers(2, 20)))
    n_transient = int(g.integers(0, 6))
    n_cache = max(1, max_n - n_transient + int(g.integers(0, 30)))
    admit = int(g.integers(0, 4)) * 2
    calls = _trace(seed, n_layers, n_routed, 60, max_n, hot=min(5, n_routed))
    ref = _run_ref(n_layers, n_routed, n_cache, n_transient, admit, calls)
    lib = moe.moe_cache_simulate(n_layers, n_routed, n_cache, n_transient, admit, calls)
    for i, (a, b) in enumerate(zip(ref, lib)):
        assert tuple(a) == tuple(b), (seed, i, calls[i])


def test_library_policy_rejects_what_does_not_fit():
    import router_top_bucket_amd as moe
    with pytest.raises(moe.MoeError):
        moe.moe_cache_simulate(1, 20, 2, 3, 0, [(0, list(range(6)), [1] * 6)])
    with pytest.raises(moe.MoeError):
        moe.moe_cache_simulate(1, 20, 4, 0, 0, [(1, [0], [1])])  # no such layer
