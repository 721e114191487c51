"""Pins for the oracle's masked softmax attention (CPU only).

The attention arithmetic is pinned against torch's scaled_dot_product_attention
in float64 on the CPU (a library routine the oracle does not use), against a
pure-Python brute force on tiny inputs, and against properties the pages
state: candidates are independent of each other, one pass with the modified
mask equals separate causal passes (HSTU appendix H), outputs depend only on
time differences, and a fully masked row gives zero.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from rk_workloads import (CANDIDATE, DAY, HISTORY, NOW, PROFILE, REALTIME, make_config,
                          make_custom, random_layout)

ROPE = dict(phi_min=1e-4, dt_max=31_536_000.0, base=6e5)


def _sdpa(q, k, v, mask=None, causal=False):
    """torch SDPA on [L, H, d] float64 CPU tensors."""
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, is_causal=causal)
    return o.numpy().transpose(1, 0, 2)


def _run(wl, **kw):
    args = dict(delay=wl.delay, window=wl.window, static_bidirectional=wl.static_bidirectional)
    args.update(kw)
    return oracle.attention_forward(wl.req_offsets, wl.seg_kind, wl.timestamps,
                                    wl.q.astype(np.float64), wl.k.astype(np.float64),
                                    wl.v.astype(np.float64), **args)


def test_causal_equals_sdpa():
    rng = np.random.default_rng(11)
    L = 70
    wl = make_custom([[(HISTORY, np.sort(rng.integers(NOW - 10**6, NOW, size=L)))]],
                     heads=3, d_head=16, seed=5)
    o, lse = _run(wl)
    ref = _sdpa(wl.q.astype(np.float64), wl.k.astype(np.float64), wl.v.astype(np.float64),
                causal=True)
    assert np.allclose(o, ref, atol=1e-12, rtol=0)


def test_equal_timestamps_rope_reduces_to_sdpa():
    """All tokens at the same time: every pair is rotated by the same angle, so
    scores are those of the unrotated vectors."""
    L = 33
    wl = make_custom([[(HISTORY, np.full(L, NOW, np.int64))]], heads=2, d_head=32, seed=6)
    o, _ = _run(wl, rope=ROPE)
    ref = _sdpa(wl.q.astype(np.float64), wl.k.astype(np.float64), wl.v.astype(np.float64),
                causal=True)
    assert np.allclose(o, ref, atol=1e-11, rtol=0)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_general_masks_equal_sdpa_with_explicit_mask(seed):
    rng = np.random.default_rng(seed)
    reqs = random_layout(rng, 3, 60)
    for bidir, delay, window in ((True, 0, 0), (False, 3600, 0), (False, 0, 5), (False, 7200, 9)):
        wl = make_custom(reqs, heads=2, d_head=8, seed=seed, delay=delay, window=window,
                         static_bidirectional=bidir)
        o, lse = _run(wl, rope=ROPE)
        for r in range(wl.num_requests):
            a, b = wl.request(r)
            if b == a:
                continue
            vis = oracle.visibility(wl.seg_kind[a:b], wl.timestamps[a:b], delay=delay,
                                    window=window, static_bidirectional=bidir)
            qr = oracle.time_rope(wl.q[a:b].astype(np.float64), wl.timestamps[a:b], **ROPE)
            kr = oracle.time_rope(wl.k[a:b].astype(np.float64), wl.timestamps[a:b], **ROPE)
            ref = _sdpa(qr, kr, wl.v[a:b].astype(np.float64), mask=vis)
            has = vis.any(axis=1)
            assert np.allclose(o[a:b][has], ref[has], atol=1e-12, rtol=0)
            assert np.all(o[a:b][~has] == 0.0)
            assert np.all(np.isneginf(lse[:, a:b][:, ~has]))


def test_brute_force_tiny():
    """Pure-Python per-pair loops, no numpy in the arithmetic."""
    rng = np.random.default_rng(21)
    reqs = [[(PROFILE, np.full(2, NOW - 500, np.int64)),
             (HISTORY, np.array([NOW - 400, NOW - 300, NOW - 290, NOW - 100])),
             (REALTIME, np.array([NOW - 50, NOW - 20, NOW - 20])),
             (CANDIDATE, np.array([NOW - 30, NOW, NOW - 60]))]]
    for bidir, delay, window in ((True, 0, 0), (False, 60, 0), (False, 0, 2)):
        wl = make_custom(reqs, heads=1, d_head=4, seed=8, delay=delay, window=window,
                         static_bidirectional=bidir)
        o, lse = _run(wl, rope=ROPE)
        seg = [int(x) for x in wl.seg_kind]
        ts = [int(x) for x in wl.timestamps]
        L, d = len(seg), 4
        w = [ROPE["phi_min"] / ROPE["dt_max"] * ROPE["base"] ** (2 * i / d) for i in range(d // 2)]

        def rot(x, t):
            y = list(x)
            for i in range(d // 2):
                a = t * w[i]
                y[2 * i] = x[2 * i] * math.cos(a) - x[2 * i + 1] * math.sin(a)
                y[2 * i + 1] = x[2 * i] * math.sin(a) + x[2 * i + 1] * math.cos(a)
            return y

        def sees(i, j):
            st = lambda s: s in (PROFILE, HISTORY)
            if seg[j] == CANDIDATE:
                return i == j
            if st(seg[i]) and st(seg[j]):
                if bidir:
                    return True
                ok = j <= i
                if window:
                    ok = ok and i - j < window
                if delay:
                    ok = ok and not (ts[j] > ts[i] - delay)
                return ok
            if st(seg[i]):
                return False
            if seg[i] == REALTIME:
                return st(seg[j]) or (j <= i and ts[j] <= ts[i])
            return st(seg[j]) or ts[j] < ts[i]

        Q = [rot([float(x) for x in wl.q[i, 0]], ts[i]) for i in range(L)]
        K = [rot([float(x) for x in wl.k[i, 0]], ts[i]) for i in range(L)]
        V = [[float(x) for x in wl.v[i, 0]] for i in range(L)]
        for i in range(L):
            keys = [j for j in range(L) if sees(i, j)]
            if not keys:
                assert all(x == 0.0 for x in o[i, 0])
                continue
            sc = {j: sum(Q[i][c] * K[j][c] for c in range(d)) / math.sqrt(d) for j in keys}
            mx = max(sc.values())
            den = sum(math.exp(s - mx) for s in sc.values())
            out = [sum(math.exp(sc[j] - mx) * V[j][c] for j in keys) / den for c in range(d)]
            assert np.allclose(o[i, 0], out, atol=1e-13)
            assert lse[0, i] == pytest.approx(mx + math.log(den), abs=1e-13)


def test_single_visible_key_gives_value_row():
    """A row with exactly one visible key returns that key's value and a
    log-sum-exp equal to the scaled score."""
    wl = make_config(1)
    o, lse = _run(wl, rope=ROPE)
    vis = oracle.visibility(wl.seg_kind, wl.timestamps, delay=wl.delay, window=0,
                            static_bidirectional=False)
    rows = np.nonzero(vis.sum(axis=1) == 1)[0]
    assert rows.shape[0] > 0
    for i in rows:
        j = int(np.nonzero(vis[i])[0][0])
        assert np.allclose(o[i], wl.v[j].astype(np.float64), atol=1e-14)


def test_fully_masked_rows_zero_and_lse_neg_inf():
    wl = make_config(1)
    o, lse = _run(wl, rope=ROPE)
    assert np.all(o[0] == 0.0)
    assert np.all(np.isneginf(lse[:, 0]))
    vis = oracle.visibility(wl.seg_kind, wl.timestamps, delay=wl.delay, window=0,
                            static_bidirectional=False)
    assert np.array_equal(np.isfinite(lse[0]), vis.any(axis=1))


def test_time_shift_invariance_full_forward():
    """Shift all timestamps (and the delay rule's inputs) by a constant: the
    mask is unchanged (differences only) and RoPE scores depend only on
    differences, so outputs are unchanged."""
    wl = make_config(1)
    o0, l0 = _run(wl, rope=ROPE)
    for shift in (10**9, -NOW, 987_654.321):
        o1, l1 = oracle.attention_forward(
            wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q, wl.k, wl.v, delay=wl.delay,
            window=0, static_bidirectional=False, rope=ROPE,
            rope_times=wl.timestamps.astype(np.float64) + shift)
        assert np.allclose(o1, o0, atol=1e-10, rtol=0)
        fin = np.isfinite(l0)
        assert np.array_equal(fin, np.isfinite(l1))
        assert np.allclose(l1[fin], l0[fin], atol=1e-10)


def test_candidates_independent_and_permutation_equivariant():
    rng = np.random.default_rng(4)
    hist = np.sort(rng.integers(NOW - 10**6, NOW - DAY, size=40))
    rt = np.sort(rng.integers(NOW - DAY, NOW, size=7))
    cand = rng.integers(NOW - DAY, NOW, size=6)
    reqs = [[(PROFILE, np.full(3, NOW, np.int64)), (HISTORY, hist), (REALTIME, rt),
             (CANDIDATE, cand)]]
    wl = make_custom(reqs, heads=2, d_head=8, seed=9, static_bidirectional=True)
    o, _ = _run(wl, rope=ROPE)
    n0 = 3 + 40 + 7
    perm = rng.permutation(6)
    idx = np.concatenate([np.arange(n0), n0 + perm])
    wp = make_custom([[(PROFILE, np.full(3, NOW, np.int64)), (HISTORY, hist), (REALTIME, rt),
                       (CANDIDATE, cand[perm])]], heads=2, d_head=8, seed=9,
                     static_bidirectional=True)
    wp.q, wp.k, wp.v = wl.q[idx], wl.k[idx], wl.v[idx]
    op, _ = _run(wp, rope=ROPE)
    assert np.allclose(op, o[idx], atol=1e-13)
    # changing one candidate's q/k/v leaves every other row unchanged
    wc = make_custom(reqs, heads=2, d_head=8, seed=9, static_bidirectional=True)
    wc.q, wc.k, wc.v = wl.q.copy(), wl.k.copy(), wl.v.copy()
    wc.q[n0 + 2] += 3.0
    wc.k[n0 + 2] -= 2.0
    wc.v[n0 + 2] *= -1.0
    oc, _ = _run(wc, rope=ROPE)
    keep = np.ones(n0 + 6, dtype=bool)
    keep[n0 + 2] = False
    assert np.array_equal(oc[keep], o[keep])


def test_mfalcon_one_pass_equals_separate_causal_passes():
    """HSTU appendix H: with the modified mask, each target's output equals a
    separate standard causal pass over [history, that target]."""
    rng = np.random.default_rng(12)
    n_hist, b_m = 24, 5
    hist = np.sort(rng.integers(NOW - 10**6, NOW - 10, size=n_hist))
    cand = np.full(b_m, NOW, np.int64)
    wl = make_custom([[(HISTORY, hist), (CANDIDATE, cand)]], heads=2, d_head=16, seed=13)
    o, _ = _run(wl, rope=ROPE)
    for c in range(b_m):
        idx = np.concatenate([np.arange(n_hist), [n_hist + c]])
        qr = oracle.time_rope(wl.q[idx].astype(np.float64), wl.timestamps[idx], **ROPE)
        kr = oracle.time_rope(wl.k[idx].astype(np.float64), wl.timestamps[idx], **ROPE)
        ref = _sdpa(qr, kr, wl.v[idx].astype(np.float64), causal=True)
        assert np.allclose(o[n_hist + c], ref[-1], atol=1e-12)


def test_attention_rows_matches_forward():
    wl = make_config(1)
    o, lse = _run(wl, rope=ROPE)
    toks = np.array([0, 5, 100, 255, 256, 271])
    for h in range(2):
        orow, lrow = oracle.attention_rows(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q, wl.k,
                                           wl.v, toks, h, delay=wl.delay, window=0,
                                           static_bidirectional=False, rope=ROPE)
        assert np.allclose(orow, o[toks, h], atol=1e-13)
        fin = np.isfinite(lse[h, toks])
        assert np.allclose(lrow[fin], lse[h, toks][fin], atol=1e-13)
