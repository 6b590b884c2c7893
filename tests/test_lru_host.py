"""The library's host-side slot policy (edge0_lru_*) against the oracle's
LRU replay, request by request: slots, hits and evicted keys bit-exact, on
the hand traces and on Zipf routing traces in the canonical orders of both
staging arms (prediction arm with the heads flushed after the last layer;
on-demand arm).  Runs on the CPU: the policy does no device work."""
import os

import numpy as np
import pytest

import oracle as O
from synth import gen as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def E():
    from int4_expert_streaming_amd import edge0
    return edge0


def _drive(E, events, ids_of, n_slots, n_layers, n_experts):
    """Feeds the oracle's event list to edge0_lru; returns the records in the
    oracle's form plus the library's totals."""
    lru = E.Lru(n_slots, n_layers, n_experts)
    recs = []
    for kind, L, t in events:
        if kind == "use":
            lru.release(L, t)
            continue
        ids = [int(e) for e in ids_of(L, t)]
        slots, hit, ev = lru.request(L, t, ids)
        recs.append({"L": L, "t": t, "ids": ids, "slots": slots.tolist(),
                     "hit": [bool(h) for h in hit],
                     "evicted": [None if k < 0 else (int(k) // n_experts, int(k) % n_experts)
                                 for k, h in zip(ev, hit) if not h]})
    st = lru.stats()
    lru.close()
    return recs, st


def _oracle(events, ids_of, n_slots):
    recs, tot = O.lru_replay(events, ids_of, n_slots)
    for r in recs:
        r["evicted"] = [None if k is None else tuple(k) for k in r["evicted"]]
    return recs, tot


@pytest.mark.parametrize("arm", ["ahead", "demand"])
@pytest.mark.parametrize("n_slots", [28, 40, 97, 160])
def test_lru_matches_oracle_tiny_stack(E, arm, n_slots):
    Lc, T, En, K = 10, 24, 16, 4
    trace = G.zipf_trace(En, K, Lc, T + 1, seed=7, keep_p=0.1)
    if arm == "ahead":
        ev = O.canonical_requests(T, Lc, range(2, 8), range(3, 9), heads_at_end=True)
    else:
        ev = O.canonical_requests(T, Lc, range(0), range(0))
    ids_of = lambda L, t: trace[t, L]
    want, tot = _oracle(ev, ids_of, n_slots)
    got, st = _drive(E, ev, ids_of, n_slots, Lc, En)
    assert got == want
    assert (st["hits"], st["misses"], st["touches"]) == (tot["hits"], tot["misses"], tot["touches"])
    assert st["evictions"] == sum(k is not None for r in want for k in r["evicted"])
    assert st["requests"] == len(want)


def test_lru_matches_oracle_qwen3moe_stack(E):
    """The 40-layer stack's pool: 3 GiB of 2,924,544-byte bundles = 1,101
    slots, K = 4, 128 experts, both arms, 24 steps."""
    Lc, T, En, K = 40, 24, 128, 4
    n_slots = (3 << 30) // 2_924_544
    assert n_slots == 1101
    trace = G.zipf_trace(En, K, Lc, T + 1, seed=0, keep_p=0.06)
    ids_of = lambda L, t: trace[t, L]
    for ev in (O.canonical_requests(T, Lc, range(6, 38), range(7, 39), heads_at_end=True),
               O.canonical_requests(T, Lc, range(0), range(0))):
        want, tot = _oracle(ev, ids_of, n_slots)
        got, st = _drive(E, ev, ids_of, n_slots, Lc, En)
        assert got == want
        assert st["misses"] == tot["misses"]


def test_lru_hand_traces_through_library(E):
    """The hand-traced cases of the golden file, replayed by the library."""
    from tests.test_oracle_pins import _lru_cases
    for name, case in _lru_cases().items():
        events, sets, want = [], {}, []
        for row in case["ev"]:
            L, t = int(row[1]), int(row[2])
            if row[0] == "use":
                events.append(("use", L, t))
                continue
            bar = row.index("|")
            bar2 = row.index("|", bar + 1)
            sets[(L, t)] = [int(v) for v in row[3:bar]]
            want.append(([int(v) for v in row[bar + 1:bar2]], [v == "1" for v in row[bar2 + 1:]]))
            events.append(("req", L, t))
        n_layers = 1 + max(L for _, L, _ in events)
        n_experts = 1 + max(max(v) for v in sets.values())
        got, _ = _drive(E, events, lambda L, t: sets[(L, t)], case["n"], n_layers, n_experts)
        assert [(r["slots"], r["hit"]) for r in got] == want, name


def test_lru_no_slot_leaves_state_unchanged(E):
    """Every slot pinned: EDGE0_ENOSLOT, and the pool answers the next
    request exactly as if the refused one had not been made."""
    lru = E.Lru(2, 1, 8)
    lru.request(0, 0, [1, 2])
    with pytest.raises(E.Edge0Error) as ei:
        lru.request(0, 1, [3])
    assert ei.value.code == E.EDGE0_ENOSLOT
    lru.release(0, 0)
    slots, hit, ev = lru.request(0, 1, [3])
    assert slots.tolist() == [0] and hit.tolist() == [0] and ev.tolist() == [1]
    assert lru.stats()["requests"] == 2


def test_lru_rejects_bad_requests(E):
    lru = E.Lru(4, 2, 8)
    for args in ((0, 0, [8]), (0, 0, [-1]), (2, 0, [1]), (0, 0, [1, 1]), (0, -1, [1]),
                 (0, 0, list(range(17)))):
        with pytest.raises(E.Edge0Error) as ei:
            lru.request(*args)
        assert ei.value.code == E.EDGE0_EINVAL
    lru.request(0, 0, [1])
    with pytest.raises(E.Edge0Error):
        lru.request(0, 0, [2])      # (layer, step) already pending
    with pytest.raises(E.Edge0Error):
        lru.release(1, 0)           # not pending
    assert lru.stats()["requests"] == 1
