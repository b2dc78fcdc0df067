"""The expert-cache reference model (oracle/cache_model.py) against facts
that do not come from it: a textbook LRU fault count, an independent
recency-list LRU, the inclusion property of LRU, and the invariants the
library documents for pinning and replacement."""
import collections
import random

from oracle.cache_model import ExpertCacheModel


def test_textbook_lru_fault_count():
    # Silberschatz, Galvin & Gagne, "Operating System Concepts", LRU page
    # replacement: this reference string with three frames gives 12 faults.
    ref = [7, 0, 1, 2, 0, 3, 0, 4, 2, 3, 0, 3, 2, 1, 2, 0, 1, 7, 0, 1]
    m = ExpertCacheModel(8, 3)
    for e in ref:
        m.step([e])
    assert m.misses == 12
    assert m.hits == len(ref) - 12
    assert m.resident() == {0, 1, 7}


def _recency_lru(ref, S):
    """Classic LRU over a recency list: (misses, resident set)."""
    od = collections.OrderedDict()
    misses = 0
    for e in ref:
        if e in od:
            od.move_to_end(e)
            continue
        misses += 1
        if len(od) == S:
            od.popitem(last=False)
        od[e] = True
    return misses, set(od)


def test_single_expert_calls_match_a_recency_list_lru():
    rng = random.Random(5)
    for S in (1, 2, 5, 9):
        for _ in range(20):
            ref = [rng.randrange(16) for _ in range(60)]
            m = ExpertCacheModel(16, S)
            for e in ref:
                m.step([e])
            misses, res = _recency_lru(ref, S)
            assert m.misses == misses
            assert m.resident() == res


def test_lru_inclusion_property():
    # LRU is a stack algorithm: with one reference per call, the resident set
    # of a cache of S slots is contained in that of S+1 slots at every step
    # (so the hit count never falls as slots are added).
    rng = random.Random(11)
    ref = [min(int(rng.paretovariate(1.1)), 31) for _ in range(400)]
    models = [ExpertCacheModel(32, S) for S in range(1, 12)]
    for e in ref:
        for m in models:
            m.step([e])
        for a, b in zip(models, models[1:]):
            assert a.resident() <= b.resident()
    hits = [m.hits for m in models]
    assert hits == sorted(hits)


def _check_invariants(m: ExpertCacheModel):
    for s, e in enumerate(m.expert_of):
        if e >= 0:
            assert m.slot_of[e] == s
    for e, s in enumerate(m.slot_of):
        if s >= 0:
            assert m.expert_of[s] == e
    assert all(m.last_use[s] <= m.clock for s in range(m.S))


def test_multi_expert_calls_keep_the_batch_resident():
    rng = random.Random(3)
    E, S, k = 32, 12, 4
    m = ExpertCacheModel(E, S)
    unique = 0
    for _ in range(200):
        T = rng.choice([1, 2, 3])
        pairs = [rng.randrange(E) if rng.random() > 0.1 else -1 for _ in range(T * k)]
        m.step(pairs)
        unique += len({e for e in pairs if e >= 0})
        _check_invariants(m)
        need = {e for e in pairs if e >= 0}
        assert need <= m.resident()  # min(E, T*k) <= S, so every expert fits
        assert all(m.last_use[m.slot_of[e]] == m.clock for e in need)
        assert len(m.copies) == len({e for e, _ in m.copies})
    assert m.error == 0
    assert m.hits + m.misses == unique


def test_usage_counts_pairs_and_repin_protects_the_hot_set():
    E, S = 16, 6
    m = ExpertCacheModel(E, S)
    # experts 3 and 5 dominate the usage
    for _ in range(10):
        m.step([3, 5, 3])
    assert m.use_count[3] == 20 and m.use_count[5] == 10
    m.repin(2)
    assert sum(m.pinned) == 2
    assert {m.expert_of[s] for s in range(S) if m.pinned[s]} == {3, 5}
    # a long run of other experts never evicts the pinned pair
    for e in [0, 1, 2, 4, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15] * 3:
        m.step([e])
        assert {3, 5} <= m.resident()
    _check_invariants(m)
    # repin to a different hot set: the old pins are released
    for _ in range(50):
        m.step([9])
    m.repin(1)
    assert [m.expert_of[s] for s in range(S) if m.pinned[s]] == [9]


def test_overfull_call_sets_the_error_bit():
    m = ExpertCacheModel(8, 3)
    m.step([0, 1, 2, 3])
    assert m.error == 1
    assert m.resident() == {0, 1, 2}
