"""Pins for the sliding window with anchors (on-device page: keep the 1536
most recent tokens and the first 64 as anchors) and its ring storage."""
import numpy as np
import pytest


def _simulate_eviction(t: int, n_anchor: int, window: int) -> list[int]:
    """Replay appends 0..t into a store that, whenever it holds more than
    n_anchor + window tokens, drops the oldest non-anchor token."""
    kept: list[int] = []
    for p in range(t + 1):
        kept.append(p)
        if len(kept) > n_anchor + window:
            for i, q in enumerate(kept):
                if q >= n_anchor:
                    del kept[i]
                    break
    return kept


@pytest.mark.parametrize("A,W", [(64, 1536), (4, 8), (0, 5), (3, 1)])
def test_attended_set_equals_eviction_replay(oq, A, W):
    ts = list(range(0, 3 * (A + W) + 5))
    if len(ts) > 200:  # the page's shape: every edge, then a sparse sweep
        edges = {0, A - 1, A, A + 1, A + W - 1, A + W, A + W + 1, 2 * (A + W), 3 * (A + W) + 4}
        ts = sorted({t for t in edges if t >= 0} | set(range(0, len(ts), 397)))
    for t in ts + [32767]:
        want = _simulate_eviction(t, A, W) if t < 5000 else None
        got = oq.attended_positions(t, A, W).tolist()
        if want is not None:
            assert got == want, (A, W, t)
        assert len(got) == min(t + 1, A + W)


def test_full_context_attends_everything(oq):
    assert oq.attended_positions(10, 0, 0).tolist() == list(range(11))


def test_page_shape_at_32k(oq):
    got = oq.attended_positions(32767, 64, 1536)
    assert got.size == 1600
    assert got[:64].tolist() == list(range(64))
    assert got[64:].tolist() == list(range(32768 - 1536, 32768))


@pytest.mark.parametrize("A,W", [(64, 1536), (4, 8), (0, 5), (2, 1)])
def test_ring_slots_hold_the_attended_set(oq, A, W):
    """Writing every position p to slot_of(p) leaves exactly the attended
    positions in the A + W slots, each in its own slot."""
    ring = {}
    for t in range(0, 4 * (A + W) + 3):
        ring[oq.slot_of(t, A, W)] = t
        assert all(0 <= s < A + W for s in ring)
        assert sorted(ring.values()) == oq.attended_positions(t, A, W).tolist()


def test_linear_slots(oq):
    assert [oq.slot_of(p, 0, 0) for p in range(5)] == list(range(5))
