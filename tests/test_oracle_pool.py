"""The oracle's process pool (oracle/pool.py) reassembles the serial oracle:
its pieces tile every output row of every sequence and KV group, and the
per-sequence inputs its workers draw are the ones the tests draw."""

import dataclasses

import numpy as np

import oracle
from oracle import pool as opool
from synthetic import WORKLOADS, gen_decode_cache_b, gen_decode_query, gen_prefill


def test_prefill_pieces_equal_serial_oracle():
    over = (("L", 300), ("B", 2))
    w = dataclasses.replace(WORKLOADS["c5"], L=300, B=2)   # boosted rows included
    q, k, v = gen_prefill(w)
    want = oracle.prefill(q, k, v, scale=w.scale)
    got = np.full(want.shape, np.nan)
    tasks = opool.prefill_tasks("c5", over, rows_per_piece=64)
    assert len(tasks) == 2 * w.h_kv * 5
    with opool.oracle_pool(2) as pool:
        for b, u, r0, r1, blk in opool.prefill_pieces(pool, tasks):
            got[b, r0:r1, u * w.g:(u + 1) * w.g] = blk
        dec = dict(opool.decode_pieces(pool, "c3", (("L", 200), ("B", 3))))
    assert np.max(np.abs(got - want)) <= 1e-12
    wd = dataclasses.replace(WORKLOADS["c3"], L=200, B=3)
    qh = gen_decode_query(wd)
    kc = np.stack([gen_decode_cache_b(wd, b)[0] for b in range(3)])
    vc = np.stack([gen_decode_cache_b(wd, b)[1] for b in range(3)])
    want_d = oracle.decode(qh, kc, vc, wd.L, wd.q_pos, scale=wd.scale)
    assert sorted(dec) == [0, 1, 2]
    assert np.max(np.abs(np.stack([dec[b] for b in range(3)]) - want_d)) <= 1e-12


def test_comparison_statistics():
    cmp = opool.Comparison()
    want = np.array([[3.0, 4.0]])
    cmp.add(np.array([[3.0, 4.5]]), want, "a")
    cmp.add(np.array([[np.nan, 0.0]]), np.array([[1.0, 0.0]]), "b")
    assert cmp.max_abs == 0.5 and cmp.worst == "a"
    assert cmp.nonfinite == 1
    assert abs(cmp.rel_l2 - 0.5 / np.sqrt(26.0)) < 1e-15


def test_pool_leaves_no_process_behind():
    """After the pools close, stopping the semaphore helper of the "spawn"
    start method leaves this process without children; a later pool works
    and starts its own helper."""
    import psutil

    def one_pool():
        with opool.oracle_pool(2) as pool:
            return dict(opool.decode_pieces(pool, "c3", (("L", 64), ("B", 2))))

    assert sorted(one_pool()) == [0, 1]
    opool.stop_resource_tracker()
    assert psutil.Process().children(recursive=True) == []
    assert sorted(one_pool()) == [0, 1]
    assert opool.stop_resource_tracker()
    assert not opool.stop_resource_tracker()   # nothing left to stop
    assert psutil.Process().children(recursive=True) == []
