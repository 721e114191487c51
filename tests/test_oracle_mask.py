"""Pins for the oracle's visibility rule (CPU only).

Each test compares the oracle's explicit mask with something fixed outside
the oracle: a worked example printed on a page, a mask built from another
page's own formulation (M-FALCON, LazFormer eq. 19-21), or an exact pair
count in closed form.
"""

import json
import os

import numpy as np
import pytest

import oracle
from rk_workloads import CANDIDATE, HISTORY, NOW, PROFILE, REALTIME, make_config, make_custom

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_cadet_delay_worked_example():
    g = _load("cadet_delay_example.json")
    seg = np.full(len(g["timestamps_s"]), HISTORY, np.uint8)
    vis = oracle.visibility(seg, np.array(g["timestamps_s"]), delay=g["delay_s"], window=0,
                            static_bidirectional=False)
    assert vis.astype(int).tolist() == g["expected_visible"]


def test_mtgr_mixed_mask_example():
    g = _load("mtgr_mixed_mask_example.json")
    vis = oracle.visibility(np.array(g["seg_kind"], np.uint8), np.array(g["timestamps"]),
                            delay=0, window=0, static_bidirectional=g["static_bidirectional"])
    assert vis.astype(int).tolist() == g["expected_visible"]


@pytest.mark.parametrize("n_c,b_m", [(3, 4), (5, 1), (1, 6)])
def test_mfalcon_modified_lower_triangle(n_c, b_m):
    """HSTU appendix H: a (2n_c + b_m) lower-triangular mask with entries
    i, j >= 2n_c, i != j removed, built here from that description."""
    n = 2 * n_c + b_m
    ref = np.tril(np.ones((n, n), dtype=bool))
    for i in range(2 * n_c, n):
        for j in range(2 * n_c, n):
            if i != j:
                ref[i, j] = False
    seg = np.array([HISTORY] * (2 * n_c) + [CANDIDATE] * b_m, np.uint8)
    ts = np.arange(n, dtype=np.int64) + NOW
    vis = oracle.visibility(seg, ts, delay=0, window=0, static_bidirectional=False)
    assert np.array_equal(vis, ref)


@pytest.mark.parametrize("Lt,N,W", [(10, 3, 4), (7, 2, 1), (9, 4, 20), (16, 5, 3)])
def test_lazformer_eq19_21(Lt, N, W):
    """LazFormer section 2.3, eq. 19-21 with no global-tail queries (G = 0),
    1-based p, q exactly as printed."""
    n = Lt + N
    ref = np.zeros((n, n), dtype=bool)
    for p in range(1, n + 1):
        for q in range(1, n + 1):
            if p <= Lt and q <= Lt and q <= p and (p - q < W):
                ref[p - 1, q - 1] = True
            elif p > Lt and q <= Lt:
                ref[p - 1, q - 1] = True
            elif p > Lt and q > Lt and p == q:
                ref[p - 1, q - 1] = True
    seg = np.array([HISTORY] * Lt + [CANDIDATE] * N, np.uint8)
    ts = np.arange(n, dtype=np.int64) + NOW
    vis = oracle.visibility(seg, ts, delay=0, window=W, static_bidirectional=False)
    assert np.array_equal(vis, ref)


@pytest.mark.parametrize("Lt,N,W,G", [(12, 3, 4, 3), (30, 5, 7, 10), (20, 0, 1, 20),
                                      (25, 4, 6, 0), (9, 2, 3, 1)])
def test_lazformer_eq19_21_global_tail(Lt, N, W, G):
    """LazFormer section 2.3, eq. 19-21 with G global-tail queries, built
    literally (1-based p, q): history query p sees history key q iff q <= p
    and (p - q < W or p > Lt - G); candidates see all history and
    themselves."""
    n = Lt + N
    ref = np.zeros((n, n), dtype=bool)
    for p in range(1, n + 1):
        for q in range(1, n + 1):
            if p <= Lt and q <= Lt and q <= p and (p - q < W or p > Lt - G):
                ref[p - 1, q - 1] = True
            elif p > Lt and q <= Lt:
                ref[p - 1, q - 1] = True
            elif p > Lt and q > Lt and p == q:
                ref[p - 1, q - 1] = True
    seg = np.array([HISTORY] * Lt + [CANDIDATE] * N, np.uint8)
    ts = np.arange(n, dtype=np.int64) + NOW
    vis = oracle.visibility(seg, ts, delay=0, window=W, static_bidirectional=False,
                            global_tail=G)
    assert np.array_equal(vis, ref)


def test_global_tail_pair_count_closed_form():
    """History of L with window W and G global-tail queries: the first L - G
    rows see min(p + 1, W) keys, the last G rows see p + 1 keys."""
    L, W, G = 700, 64, 100
    seg = np.full(L, HISTORY, np.uint8)
    ts = np.arange(L, dtype=np.int64) + NOW
    want = sum(min(p + 1, W) for p in range(L - G)) + sum(p + 1 for p in range(L - G, L))
    got = oracle.count_visible(seg, ts, delay=0, window=W, static_bidirectional=False,
                               global_tail=G)
    assert got == want == 36384 + 65050


def test_delay_zero_no_window_is_lower_triangle_even_with_ties():
    rng = np.random.default_rng(7)
    L = 40
    ts = np.sort(rng.integers(0, 5, size=L)) + NOW  # many timestamp ties
    seg = np.full(L, HISTORY, np.uint8)
    vis = oracle.visibility(seg, ts, delay=0, window=0, static_bidirectional=False)
    assert np.array_equal(vis, np.tril(np.ones((L, L), dtype=bool)))


def test_cadet_pair_count_closed_form():
    g = _load("pair_counts.json")
    L, N = g["cadet_L"], g["cadet_N"]
    seg = np.array([HISTORY] * L + [CANDIDATE] * N, np.uint8)
    ts = np.arange(L + N, dtype=np.int64) + NOW
    n = oracle.count_visible(seg, ts, delay=0, window=0, static_bidirectional=False)
    assert n == g["cadet_masked_pairs_exact"]
    # the page's approximate figures (about 21.1 M dense vs about 10.4 M masked)
    assert abs((L + N) ** 2 - g["cadet_dense_pairs_page_approx"]) / g["cadet_dense_pairs_page_approx"] < 0.005
    assert abs(n - g["cadet_masked_pairs_page_approx"]) / g["cadet_masked_pairs_page_approx"] < 0.005
    assert abs(n - (L * L / 2 + L * N)) / n < 0.001


def test_serving_workload_pair_count_closed_form():
    g = _load("pair_counts.json")
    wl = make_config(3, with_qkv=False)
    a, b = wl.request(0)
    n = oracle.count_visible(wl.seg_kind[a:b], wl.timestamps[a:b], delay=wl.delay,
                             window=wl.window, static_bidirectional=wl.static_bidirectional)
    assert n == g["serving_per_request"]


def test_tm20k_workload_pair_count_closed_form():
    g = _load("pair_counts.json")
    wl = make_config(5, with_qkv=False)
    a, b = wl.request(3)
    n = oracle.count_visible(wl.seg_kind[a:b], wl.timestamps[a:b], delay=wl.delay,
                             window=wl.window, static_bidirectional=wl.static_bidirectional,
                             row_block=2048)
    assert n == g["tm20k_per_request"]


def test_mtgr_workload_pair_count():
    """Static 3032 bidirectional, RT causal, each target: static + RT strictly
    before it + itself."""
    wl = make_config(4, with_qkv=False)
    a, b = wl.request(0)
    seg, ts = wl.seg_kind[a:b], wl.timestamps[a:b]
    n = oracle.count_visible(seg, ts, delay=0, window=0, static_bidirectional=True)
    S = 32 + 3000
    rt = ts[seg == REALTIME]
    cand = ts[seg == CANDIDATE]
    expected = S * S + sum(S + i + 1 for i in range(200)) + sum(S + int((rt < t).sum()) + 1 for t in cand)
    assert n == expected
    # closed form without the target-to-real-time part: S^2 + sum_i (S+i+1) + 100 (S+1)
    assert n - int(sum((rt < t).sum() for t in cand)) == 10_122_824


def test_candidate_permutation_permutes_mask():
    rng = np.random.default_rng(3)
    hist = np.sort(rng.integers(NOW - 10_000, NOW - 100, size=20))
    rt = np.sort(rng.integers(NOW - 100, NOW, size=6))
    cand = rng.integers(NOW - 100, NOW, size=5)
    seg = np.array([PROFILE] * 2 + [HISTORY] * 20 + [REALTIME] * 6 + [CANDIDATE] * 5, np.uint8)
    ts = np.concatenate([[hist[0]] * 2, hist, rt, cand]).astype(np.int64)
    base = oracle.visibility(seg, ts, delay=0, window=0, static_bidirectional=True)
    perm = rng.permutation(5)
    idx = np.concatenate([np.arange(28), 28 + perm])
    vis = oracle.visibility(seg, ts[idx], delay=0, window=0, static_bidirectional=True)
    assert np.array_equal(vis, base[np.ix_(idx, idx)])


def test_first_rows_fully_masked_under_delay():
    wl = make_config(1, with_qkv=False)
    vis = oracle.visibility(wl.seg_kind, wl.timestamps, delay=wl.delay, window=0,
                            static_bidirectional=False)
    assert not vis[0].any()
    # candidates see every history token and themselves, no other candidate
    L = 256
    assert vis[L:, :L].all()
    assert np.array_equal(vis[L:, L:], np.eye(16, dtype=bool))


def test_key_subset_equals_full_matrix():
    """Rows and keys evaluated as a subset give the full matrix's entries
    (every segment kind, delay with anchor-dated and earlier profiles,
    window, global tail)."""
    from rk_workloads import random_layout
    rng = np.random.default_rng(41)
    wl = make_custom(random_layout(rng, 6, 300, allow_empty=False), heads=1, d_head=2,
                     with_qkv=False)
    for bidir, delay, window, G in ((True, 0, 0, 0), (False, 600, 0, 0), (False, 300, 25, 4)):
        for r in range(wl.num_requests):
            a, b = wl.request(r)
            seg, ts = wl.seg_kind[a:b], wl.timestamps[a:b]
            full = oracle.visibility(seg, ts, delay=delay, window=window,
                                     static_bidirectional=bidir, global_tail=G)
            rows = rng.choice(b - a, size=min(11, b - a), replace=False)
            cols = rng.choice(b - a, size=min(13, b - a), replace=False)
            sub = oracle.visible_rows(seg, ts, rows, delay=delay, window=window,
                                      static_bidirectional=bidir, global_tail=G, cols=cols)
            assert np.array_equal(sub, full[np.ix_(rows, cols)])
