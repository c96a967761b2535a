"""Pins for the LFU slot-cache simulator (CPU only)."""
import numpy as np
import pytest

from oracle.lfu import LFUCache, simulate

A, B, C, D = 10, 11, 12, 13


def test_hand_trace_two_slots():
    ev, _ = simulate([[A], [B], [A], [C], [A], [B]], n_slots=2, n_experts=16)
    assert ev == [
        [(A, 0, 0, -1)],
        [(B, 1, 0, -1)],
        [(A, 0, 1, -1)],
        [(C, 1, 0, B)],     # B has freq 1 < A's freq 2
        [(A, 0, 1, -1)],
        [(B, 1, 0, C)],
    ]


def test_equal_frequency_evicts_least_recent():
    ev, _ = simulate([[A], [B], [C]], n_slots=2, n_experts=16)
    assert ev[2] == [(C, 0, 0, A)]


def test_equal_frequency_and_recency_evicts_lowest_slot():
    # A and B arrive in the same step, so (freq, last) ties; slot index decides
    ev, _ = simulate([[A, B], [C]], n_slots=2, n_experts=16)
    assert ev[1] == [(C, 0, 0, A)]


def test_current_token_slots_are_pinned():
    # C must not evict A or B although they have lower frequency than D
    ev, _ = simulate([[D, A], [D, B], [D, A, B]], n_slots=3, n_experts=16)
    assert ev[2][0][2] == 1
    c = LFUCache(3, 16)
    c.step([D]); c.step([D]); c.step([A, B])
    out = c.step([A, B, C])
    assert out[2] == (C, 0, 0, D)


def test_events_in_rank_order_with_hits_first():
    c = LFUCache(4, 16)
    c.step([A, B])
    out = c.step([C, A, D, B])
    assert [e[0] for e in out] == [C, A, D, B]
    assert [e[2] for e in out] == [0, 1, 0, 1]
    assert out[0][1] == 2 and out[2][1] == 3


def test_enough_slots_miss_once_per_distinct_id():
    rng = np.random.default_rng(0)
    rows = [rng.choice(32, 8, replace=False) for _ in range(200)]
    _, c = simulate(rows, n_slots=32, n_experts=32)
    assert c.misses == len(set(np.concatenate(rows).tolist()))


def test_same_ids_every_token_miss_only_first_time():
    rows = [list(range(8))] * 50
    _, c = simulate(rows, n_slots=16, n_experts=128)
    assert c.misses == 8 and c.hits == 8 * 49


def test_disjoint_consecutive_sets_with_k_slots_all_miss():
    rows = [[(8 * t + j) % 128 for j in range(8)] for t in range(40)]
    _, c = simulate(rows, n_slots=8, n_experts=128)
    assert c.hits == 0 and c.misses == 8 * 40


def test_invariants_on_random_zipf_trace():
    rng = np.random.default_rng(1)
    p = np.arange(1, 129) ** -1.1
    p /= p.sum()
    c = LFUCache(16, 128)
    T = 300
    for t in range(T):
        ids = rng.choice(128, 8, replace=False, p=p)
        out = c.step(ids)
        slots = [e[1] for e in out]
        assert len(set(slots)) == 8
        for e, s, hit, ev in out:
            assert c.expert[s] == e
        assert sorted(x for x in c.expert if x >= 0) == sorted(set(x for x in c.expert if x >= 0))
    assert c.hits + c.misses == 8 * T
    assert c.hits > 0


def test_rejects_bad_ids():
    c = LFUCache(16, 128)
    with pytest.raises(ValueError):
        c.step([1, 1])
    with pytest.raises(ValueError):
        c.step([128])
    with pytest.raises(ValueError):
        LFUCache(2, 16).step([1, 2, 3])


def test_least_recent_wins_over_lower_slot_index():
    # after [A],[B],[C] slot 0 holds C (last 2) and slot 1 holds B (last 1)
    ev, _ = simulate([[A], [B], [C], [D]], n_slots=2, n_experts=16)
    assert ev[3] == [(D, 1, 0, B)]


def test_frequency_beats_recency():
    # A is used twice, B once but more recently: the miss evicts B
    ev, _ = simulate([[A], [A], [B], [C]], n_slots=2, n_experts=16)
    assert ev[3] == [(C, 1, 0, B)]


# ---------------------------------------------------------------- LRU variant
def test_lru_hand_trace_differs_from_lfu():
    # A is used twice, then B once, then C arrives: LFU evicts B (freq 1 < 2),
    # LRU evicts A (used at step 1, B at step 2)
    rows = [[A], [A], [B], [C]]
    ev_lfu, _ = simulate(rows, n_slots=2, n_experts=16)
    ev_lru, _ = simulate(rows, n_slots=2, n_experts=16, policy="lru")
    assert ev_lfu[3] == [(C, 1, 0, B)]
    assert ev_lru[3] == [(C, 0, 0, A)]


def textbook_lru(trace, capacity):
    """Hits / misses of a plain single-key LRU cache (recency list)."""
    from collections import OrderedDict
    od, hits = OrderedDict(), 0
    out = []
    for x in trace:
        if x in od:
            od.move_to_end(x)
            hits += 1
            out.append(True)
        else:
            if len(od) == capacity:
                od.popitem(last=False)
            od[x] = None
            out.append(False)
    return out, list(od.keys())


@pytest.mark.parametrize("seed,cap", [(0, 2), (1, 4), (2, 7)])
def test_lru_one_id_per_step_is_textbook_lru(seed, cap):
    rng = np.random.default_rng(seed)
    trace = [int(v) for v in rng.integers(0, 3 * cap, 400)]
    want_hit, want_resident = textbook_lru(trace, cap)
    c = LFUCache(cap, 3 * cap, policy="lru")
    got = [bool(c.step([x])[0][2]) for x in trace]
    assert got == want_hit
    assert sorted(e for e in c.expert if e >= 0) == sorted(want_resident)


def test_lru_pins_the_current_token_and_fills_empty_slots_first():
    c = LFUCache(3, 16, policy="lru")
    assert [e[1] for e in c.step([A, B])] == [0, 1]
    c.step([C])                       # the empty slot 2
    c.step([A])                       # A recent again; B now least recent
    out = c.step([B, D])              # B hits; D must not evict B although it is the oldest
    assert out[0] == (B, 1, 1, -1) and out[1] == (D, 2, 0, C)
