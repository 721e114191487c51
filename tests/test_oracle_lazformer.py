"""Pins for the oracle's LazFormer pre-passes (CPU only): group-sum history
compression (section 2.3, eq. 16-18) and the per-layer history length of
eq. 22.

* The seven compression settings of section 3.5 (table 6) give the printed
  lengths from a 2048-event history, and the default gives 1152
  (tests/golden/lazformer_lengths.json).
* eq. 22 at the default (L~ = 1152, N_min = 128) over five layers gives
  1152, 896, 640, 384, 128 (exact integers); first layer = L~, last = N_min.
* Compression by brute force on tiny inputs; sums are preserved per request
  and feature; keep >= L or group = 1 is the identity; time order and the
  newest-member timestamp of each group.
* Pruning keeps exactly the last N^l history tokens and every other token.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from rk_workloads import (CANDIDATE, HISTORY, NOW, PROFILE, REALTIME, make_custom,
                          random_layout)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lazformer_lengths.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_compression_length_table():
    g = _golden()
    L = g["history_length"]
    for row in g["compression_table"]:
        assert oracle.compressed_history_length(L, row["keep"], row["group"]) == row["length"]
    d = g["default"]
    assert oracle.compressed_history_length(L, d["keep"], d["group"]) == d["l_tilde"]


def test_compression_table_through_the_layout():
    """The same lengths come out of the full compression of one request."""
    g = _golden()
    L = g["history_length"]
    hist = np.arange(NOW - 10 * L, NOW, 10, dtype=np.int64)
    wl = make_custom([[(HISTORY, hist)]], heads=1, d_head=2, seed=1, with_qkv=False)
    x = np.arange(L, dtype=np.float64)[:, None]
    for row in g["compression_table"]:
        offs, kinds, times, y = oracle.group_sum_compress(wl.req_offsets, wl.seg_kind,
                                                          wl.timestamps, x, keep=row["keep"],
                                                          group=row["group"])
        assert offs[-1] == row["length"]
        assert y.sum() == x.sum()


def test_prune_schedule_default():
    g = _golden()
    d = g["default"]
    got = [oracle.pruned_history_length(d["l_tilde"], d["n_min"], l, 5) for l in range(1, 6)]
    assert got == g["prune_schedule_5_layers"]
    for n_layers in (2, 3, 7, 12):
        sched = [oracle.pruned_history_length(1152, 128, l, n_layers)
                 for l in range(1, n_layers + 1)]
        assert sched[0] == 1152 and sched[-1] == 128
        assert all(a >= b for a, b in zip(sched, sched[1:]))
        # the steps of a linear schedule differ by at most one after rounding
        steps = [a - b for a, b in zip(sched, sched[1:])]
        assert max(steps) - min(steps) <= 1
    # short histories are never lengthened; N_min caps from below
    assert oracle.pruned_history_length(100, 128, 3, 5) == 100
    assert oracle.pruned_history_length(5000, 128, 1, 1) == 5000


def test_round_half_away_from_zero():
    # L~ = 129, N_min = 128, 3 layers: layer 2 -> 128.5 -> 129
    assert oracle.pruned_history_length(129, 128, 2, 3) == 129
    assert oracle.pruned_history_length(131, 128, 2, 3) == 130  # 129.5 -> 130


def test_compression_brute_force_tiny():
    t = np.array([10, 20, 35, 40, 41, 50, 60], dtype=np.int64) + NOW - 1000
    reqs = [[(PROFILE, np.full(2, NOW - 2000, np.int64)), (HISTORY, t),
             (REALTIME, np.array([NOW - 5, NOW - 3])), (CANDIDATE, np.array([NOW, NOW - 1]))],
            [(HISTORY, t[:2])],
            [(CANDIDATE, np.array([NOW]))]]
    wl = make_custom(reqs, heads=1, d_head=2, seed=2, with_qkv=False)
    x = np.arange(wl.total_tokens * 3, dtype=np.float64).reshape(-1, 3)
    offs, kinds, times, y = oracle.group_sum_compress(wl.req_offsets, wl.seg_kind, wl.timestamps,
                                                      x, keep=3, group=2)
    # request 0: 7 history -> keep the last 3, the older 4 in groups (0,1), (2,3)
    hist0 = np.arange(2, 9)  # global rows of request 0's history
    exp0 = [x[0], x[1], x[hist0[0]] + x[hist0[1]], x[hist0[2]] + x[hist0[3]],
            x[hist0[4]], x[hist0[5]], x[hist0[6]], x[9], x[10], x[11], x[12]]
    exp_t0 = [NOW - 2000, NOW - 2000, t[1], t[3], t[4], t[5], t[6], NOW - 5, NOW - 3, NOW,
              NOW - 1]
    assert offs.tolist() == [0, 11, 13, 14]
    assert np.array_equal(y[:11], np.stack(exp0))
    assert times[:11].tolist() == exp_t0
    assert kinds[:11].tolist() == [PROFILE] * 2 + [HISTORY] * 5 + [REALTIME] * 2 + [CANDIDATE] * 2
    # request 1: 2 history tokens, both kept; request 2 unchanged
    assert np.array_equal(y[11:13], x[13:15]) and np.array_equal(y[13], x[15])
    # an odd count: 6 old tokens in groups of 4 -> a partial OLDEST group of 2, then 4
    offs, kinds, times, y = oracle.group_sum_compress(
        wl.req_offsets[:2], wl.seg_kind[:13], wl.timestamps[:13], x[:13], keep=1, group=4)
    assert np.array_equal(y[2], x[hist0[0]] + x[hist0[1]])
    assert np.array_equal(y[3], x[hist0[2:6]].sum(axis=0))
    assert times[2] == t[1] and times[3] == t[5]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_compression_invariants(seed):
    rng = np.random.default_rng(seed)
    wl = make_custom(random_layout(rng, 6, 200), heads=1, d_head=2, seed=seed, with_qkv=False)
    x = rng.standard_normal((wl.total_tokens, 5))
    for keep, group in ((0, 3), (7, 8), (50, 1), (10 ** 6, 4)):
        offs, kinds, times, y = oracle.group_sum_compress(wl.req_offsets, wl.seg_kind,
                                                          wl.timestamps, x, keep=keep,
                                                          group=group)
        for r in range(wl.num_requests):
            a, b = wl.request(r)
            c, e = int(offs[r]), int(offs[r + 1])
            assert np.allclose(y[c:e].sum(axis=0), x[a:b].sum(axis=0), atol=1e-12)
            n_hist = int((wl.seg_kind[a:b] == HISTORY).sum())
            n_out = int((kinds[c:e] == HISTORY).sum())
            assert n_out == oracle.compressed_history_length(n_hist, keep, group)
            # kinds stay non-decreasing, history times stay sorted
            assert np.all(np.diff(kinds[c:e].astype(int)) >= 0)
            assert np.all(np.diff(times[c:e][kinds[c:e] == HISTORY]) >= 0)
        if group == 1 or keep >= 10 ** 6:
            assert np.array_equal(y, x) and np.array_equal(times, wl.timestamps)


@pytest.mark.parametrize("seed", [3, 4])
def test_prune_keeps_last_history_and_all_others(seed):
    rng = np.random.default_rng(seed)
    wl = make_custom(random_layout(rng, 5, 300), heads=1, d_head=2, seed=seed, with_qkv=False)
    x = np.arange(wl.total_tokens, dtype=np.float64)
    l_tilde = [int((wl.seg_kind[slice(*wl.request(r))] == HISTORY).sum())
               for r in range(wl.num_requests)]
    for layer in range(1, 6):
        offs, kinds, times, y = oracle.prune_history(wl.req_offsets, wl.seg_kind, wl.timestamps,
                                                     x, l_tilde=l_tilde, n_min=16, layer=layer,
                                                     num_layers=5)
        for r in range(wl.num_requests):
            a, b = wl.request(r)
            c, e = int(offs[r]), int(offs[r + 1])
            n = oracle.pruned_history_length(l_tilde[r], 16, layer, 5)
            hist = np.arange(a, b)[wl.seg_kind[a:b] == HISTORY]
            kept = set(hist[len(hist) - min(n, len(hist)):].tolist())
            others = set(np.arange(a, b)[wl.seg_kind[a:b] != HISTORY].tolist())
            assert sorted(y[c:e].astype(int).tolist()) == sorted(kept | others)
            assert np.all(np.diff(y[c:e]) > 0)  # order preserved
