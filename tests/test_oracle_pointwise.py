"""Pins for the oracle's HSTU pointwise aggregated attention (HSTU eq. 2:
phi_2(Q K^T + rab^{p,t}) V with SiLU, rab shared by every head), CPU only.

* time buckets: hand-computed floor(log2(1 + |dt|)) values and the cap;
* rab: per-pair pure-Python sums of the two table entries;
* brute force on tiny inputs with per-pair loops and math.exp (every
  segment kind, delay, window);
* HSTU appendix H (M-FALCON): one pass with the candidate mask equals
  separate causal passes over [history, that candidate];
* linearity in V, and a row with one visible key gives SiLU(s) v_j;
* candidates are permutation equivariant and independent of each other.
"""

import math

import numpy as np

import oracle
from rk_workloads import (CANDIDATE, HISTORY, NOW, PROFILE, REALTIME, make_custom,
                          random_layout)


def test_time_bucket_values():
    table = {0: 0, 1: 1, 2: 1, 3: 2, 6: 2, 7: 3, 8: 3, 1023: 10, 1024: 10, 86399: 16,
             31_536_000: 24}
    for dt, b in table.items():
        assert oracle.time_bucket(dt, 64) == b
        assert oracle.time_bucket(-dt, 64) == b
    assert oracle.time_bucket(10 ** 9, 12) == 11


def test_rab_pairwise():
    rng = np.random.default_rng(0)
    L = 40
    t = np.sort(rng.integers(NOW - 10 ** 7, NOW, size=L))
    pb = rng.standard_normal(9)
    tb = rng.standard_normal(20)
    rab = oracle.hstu_rab(np.arange(L), t, np.arange(L), pb, tb)
    for i in range(L):
        for j in range(L):
            ref = pb[min(abs(i - j), 8)] + tb[oracle.time_bucket(int(t[i]) - int(t[j]), 20)]
            assert rab[i, j] == ref
    # powers of two around the bucket edges (float log2 must not round up)
    t2 = np.array([0, 1, 2, 3, 4, 7, 8, 2 ** 20 - 1, 2 ** 20, 2 ** 40 - 1], dtype=np.int64)
    r2 = oracle.hstu_rab(np.arange(10), t2, np.array([0]), None, np.arange(64.0))
    assert r2[0].tolist() == [float(oracle.time_bucket(int(x), 64)) for x in t2]


def test_brute_force_tiny():
    rng = np.random.default_rng(1)
    reqs = [[(PROFILE, np.full(2, NOW - 500, np.int64)),
             (HISTORY, np.array([NOW - 400, NOW - 300, NOW - 290, NOW - 100])),
             (REALTIME, np.array([NOW - 50, NOW - 20])),
             (CANDIDATE, np.array([NOW - 30, NOW, NOW - 60]))]]
    pb, tb = rng.standard_normal(5), rng.standard_normal(12)
    for bidir, delay, window in ((True, 0, 0), (False, 60, 0), (False, 0, 2)):
        wl = make_custom(reqs, heads=1, d_head=4, seed=8, delay=delay, window=window,
                         static_bidirectional=bidir)
        o = oracle.pointwise_attention_forward(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q,
                                               wl.k, wl.v, delay=delay, window=window,
                                               static_bidirectional=bidir, scale=0.5,
                                               pos_bias=pb, time_bias=tb)
        vis = oracle.visibility(wl.seg_kind, wl.timestamps, delay=delay, window=window,
                                static_bidirectional=bidir)
        L, d = wl.total_tokens, 4
        ts = [int(x) for x in wl.timestamps]
        for i in range(L):
            out = [0.0] * d
            for j in range(L):
                if not vis[i, j]:
                    continue
                x = 0.5 * sum(float(wl.q[i, 0, c]) * float(wl.k[j, 0, c]) for c in range(d))
                x += pb[min(abs(i - j), 4)] + tb[oracle.time_bucket(ts[i] - ts[j], 12)]
                w = x / (1.0 + math.exp(-x))
                for c in range(d):
                    out[c] += w * float(wl.v[j, 0, c])
            assert np.allclose(o[i, 0], out, atol=1e-12)


def test_mfalcon_one_pass_equals_separate_causal_passes():
    rng = np.random.default_rng(2)
    n_hist, b_m = 30, 6
    hist = np.sort(rng.integers(NOW - 10 ** 6, NOW - 10, size=n_hist))
    wl = make_custom([[(HISTORY, hist), (CANDIDATE, np.full(b_m, NOW, np.int64))]], heads=2,
                     d_head=8, seed=3)
    pb, tb = rng.standard_normal(50), rng.standard_normal(25)
    kw = dict(delay=0, window=0, static_bidirectional=False, scale=0.3, pos_bias=pb,
              time_bias=tb)
    o = oracle.pointwise_attention_forward(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q,
                                           wl.k, wl.v, **kw)
    for c in range(b_m):
        idx = np.concatenate([np.arange(n_hist), [n_hist + c]])
        one = make_custom([[(HISTORY, np.concatenate([hist, [NOW]]))]], heads=2, d_head=8,
                          seed=0)
        one.q, one.k, one.v = wl.q[idx], wl.k[idx], wl.v[idx]
        oc = oracle.pointwise_attention_forward(one.req_offsets, one.seg_kind, one.timestamps,
                                                one.q, one.k, one.v, **kw)
        # history rows see the same keys at the same position differences
        assert np.allclose(oc[:n_hist], o[:n_hist], atol=1e-12)
    # a candidate sits at position n_hist + c in the packed pass and at n_hist
    # in its own pass, so position biases differ; without the position table
    # the candidate rows match exactly
    kw2 = dict(kw, pos_bias=None)
    o2 = oracle.pointwise_attention_forward(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q,
                                            wl.k, wl.v, **kw2)
    for c in range(b_m):
        idx = np.concatenate([np.arange(n_hist), [n_hist + c]])
        one = make_custom([[(HISTORY, np.concatenate([hist, [NOW]]))]], heads=2, d_head=8,
                          seed=0)
        oc = oracle.pointwise_attention_forward(one.req_offsets, one.seg_kind, one.timestamps,
                                                wl.q[idx], wl.k[idx], wl.v[idx], **kw2)
        assert np.allclose(oc[-1], o2[n_hist + c], atol=1e-12)


def test_linearity_and_single_key():
    rng = np.random.default_rng(4)
    wl = make_custom(random_layout(rng, 3, 60, allow_empty=False), heads=2, d_head=8, seed=4,
                     delay=3600)
    pb, tb = rng.standard_normal(16), rng.standard_normal(30)
    kw = dict(delay=wl.delay, window=0, static_bidirectional=False, scale=0.35, pos_bias=pb,
              time_bias=tb)
    o = oracle.pointwise_attention_forward(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q,
                                           wl.k, wl.v, **kw)
    v64, q64 = wl.v.astype(np.float64), wl.q.astype(np.float64)
    o2 = oracle.pointwise_attention_forward(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q,
                                            wl.k, 2.5 * v64 - 1.0 * q64, **kw)
    o3 = oracle.pointwise_attention_forward(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q,
                                            wl.k, wl.q, **kw)
    assert np.allclose(o2, 2.5 * o - o3, atol=1e-10)
    for r in range(wl.num_requests):
        a, b = wl.request(r)
        vis = oracle.visibility(wl.seg_kind[a:b], wl.timestamps[a:b], delay=wl.delay, window=0,
                                static_bidirectional=False)
        for i in np.nonzero(vis.sum(axis=1) == 1)[0]:
            j = int(np.nonzero(vis[i])[0][0])
            for h in range(2):
                x = 0.35 * float(wl.q[a + i, h] @ wl.k[a + j, h]) + pb[min(abs(i - j), 15)] + \
                    tb[oracle.time_bucket(int(wl.timestamps[a + i]) - int(wl.timestamps[a + j]), 30)]
                assert np.allclose(o[a + i, h], x / (1 + math.exp(-x)) * wl.v[a + j, h],
                                   atol=1e-12)
        assert np.all(o[a:b][~vis.any(axis=1)] == 0.0)


def test_candidate_permutation_equivariance():
    rng = np.random.default_rng(5)
    hist = np.sort(rng.integers(NOW - 10 ** 6, NOW - 100, size=25))
    cand = rng.integers(NOW - 90, NOW, size=5)
    wl = make_custom([[(HISTORY, hist), (CANDIDATE, cand)]], heads=1, d_head=8, seed=6)
    kw = dict(delay=0, window=0, static_bidirectional=False, scale=0.4,
              time_bias=rng.standard_normal(30))
    o = oracle.pointwise_attention_forward(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q,
                                           wl.k, wl.v, **kw)
    perm = rng.permutation(5)
    idx = np.concatenate([np.arange(25), 25 + perm])
    wp = make_custom([[(HISTORY, hist), (CANDIDATE, cand[perm])]], heads=1, d_head=8, seed=6)
    op = oracle.pointwise_attention_forward(wp.req_offsets, wp.seg_kind, wp.timestamps,
                                            wl.q[idx], wl.k[idx], wl.v[idx], **kw)
    assert np.allclose(op, o[idx], atol=1e-12)


def test_rows_form_equals_full_form():
    rng = np.random.default_rng(7)
    wl = make_custom(random_layout(rng, 4, 90), heads=2, d_head=8, seed=7, delay=120, window=9)
    kw = dict(delay=wl.delay, window=wl.window, static_bidirectional=False, scale=0.3,
              pos_bias=rng.standard_normal(11), time_bias=rng.standard_normal(20))
    o = oracle.pointwise_attention_forward(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q,
                                           wl.k, wl.v, **kw)
    toks = rng.choice(wl.total_tokens, size=25, replace=False)
    for h in range(2):
        rows = oracle.pointwise_attention_rows(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q,
                                               wl.k, wl.v, toks, h, **kw)
        # the same sums, run as BLAS products of different shapes: equal up to
        # the last bits of an fp64 rounding (|o| < 100 here)
        assert np.abs(rows - o[toks, h]).max() <= 1e-13
