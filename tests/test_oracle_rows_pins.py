"""Pins for the oracle's row movement (CPU only): gather / scatter of active rows
(TensorRT-Edge-LLM "Selective State Update" page, invokeMambaStateGather /
invokeMambaStateScatter) and the in-place packing of a cohort into working
slots (Smile "Class DeltaNetStatePool" page, activateStep / scatterActive).

The packing pins fix the two rules the page states: every source is read
before any slot is written (the page's own counterexample: homes not in
ascending order, where a sequential home-to-slot copy corrupts the cohort),
and live rows of other requests in [0, B) survive a pack / unpack round trip.
"""
import numpy as np

import oracle


def _pool(rows=6, width=4):
    return np.arange(rows * width, dtype=np.float64).reshape(rows, width) + 1.0


def test_pack_reads_every_source_first():
    pool = _pool()
    orig = pool.copy()
    homes = [3, 0, 1]
    oracle.pack(pool, homes, [])
    for b, h in enumerate(homes):
        np.testing.assert_array_equal(pool[b], orig[h])
    np.testing.assert_array_equal(pool[3:], orig[3:])
    # the mistake the page warns about: a sequential copy gives slot 1 the row
    # that slot 0 received, not home 0's original row
    naive = orig.copy()
    for b, h in enumerate(homes):
        naive[b] = naive[h]
    assert not np.array_equal(naive[1], orig[0])


def test_bystander_survives_and_round_trip():
    pool = _pool(rows=7)
    orig = pool.copy()
    # requests with homes 1 and 2 are live but not in the cohort (rows in [0, B)
    # that are neither homes nor live hold nothing and may be overwritten)
    homes, bystanders = [5, 0, 4], [1, 2]
    saved = oracle.pack(pool, homes, bystanders)
    np.testing.assert_array_equal(pool[2], orig[4])
    oracle.unpack(pool, homes, bystanders, saved)
    np.testing.assert_array_equal(pool, orig)   # an unmodified round trip changes nothing


def test_forward_results_go_home():
    pool = _pool(rows=7)
    orig = pool.copy()
    homes, bystanders = [6, 1, 0], [2]
    saved = oracle.pack(pool, homes, bystanders)
    pool[:3] += 100.0                           # the forward updates the working slots
    oracle.unpack(pool, homes, bystanders, saved)
    for h in homes:
        np.testing.assert_array_equal(pool[h], orig[h] + 100.0)
    for r in (2, 3, 4, 5):
        np.testing.assert_array_equal(pool[r], orig[r])


def test_cohort_already_in_place_copies_nothing():
    pool = _pool()
    orig = pool.copy()
    oracle.pack(pool, [0, 1, 2], [])
    np.testing.assert_array_equal(pool, orig)


def test_gather_scatter():
    pool = _pool()
    idx = np.array([4, -1, 0], dtype=np.int32)
    act = oracle.gather(pool, idx)
    np.testing.assert_array_equal(act[0], pool[4])
    np.testing.assert_array_equal(act[1], 0.0)
    np.testing.assert_array_equal(act[2], pool[0])
    res = np.zeros_like(pool)
    oracle.scatter(act + 1.0, res, idx)
    np.testing.assert_array_equal(res[4], pool[4] + 1.0)
    np.testing.assert_array_equal(res[0], pool[0] + 1.0)
    assert np.all(res[[1, 2, 3, 5]] == 0.0)
