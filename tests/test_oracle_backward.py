"""Pins for the oracle's attention backward (CPU only).

The gradients the oracle derives by the chain rule are checked against
what does not depend on that derivation:
  * torch autograd through scaled_dot_product_attention with the explicit
    boolean mask, in float64 (a library routine the oracle does not use);
  * central finite differences of the oracle's forward loss sum(dO * O),
    through time RoPE, on tiny inputs;
  * closed forms: a row that sees only itself has O = V_i, so dV = dO and
    dQ = dK = 0; a row that sees nothing and a key that nobody sees get
    zero gradients;
  * invariants of the forward: translating every rotated key by one vector
    leaves every row's softmax unchanged (sum_j R_j dK_j = 0); translating
    every value by c moves each non-empty row's output by c
    (sum_j dV_j = sum of dO over non-empty rows); scores are bilinear in q
    and k (sum q.dq = sum k.dk); a uniform time shift changes no gradient.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from rk_workloads import (CANDIDATE, HISTORY, NOW, PROFILE, REALTIME, draw_grad, make_config,
                          make_custom, random_layout)

ROPE = dict(phi_min=1e-4, dt_max=31_536_000.0, base=6e5)


def _mask_args(wl):
    return dict(delay=wl.delay, window=wl.window, static_bidirectional=wl.static_bidirectional,
                global_tail=wl.global_tail)


def _fwd(wl, q, k, v, **kw):
    o, _ = oracle.attention_forward(wl.req_offsets, wl.seg_kind, wl.timestamps, q, k, v,
                                    **_mask_args(wl), **kw)
    return o


def _bwd(wl, do, **kw):
    return oracle.attention_backward(wl.req_offsets, wl.seg_kind, wl.timestamps,
                                     wl.q.astype(np.float64), wl.k.astype(np.float64),
                                     wl.v.astype(np.float64), do.astype(np.float64),
                                     **_mask_args(wl), **kw)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_backward_equals_torch_autograd(seed):
    """delay = 0 keeps every row non-empty (each token sees itself), so SDPA's
    boolean-mask path is well defined for every row."""
    rng = np.random.default_rng(seed)
    reqs = random_layout(rng, 3, 50)
    for bidir, window in ((True, 0), (False, 0), (False, 6)):
        wl = make_custom(reqs, heads=2, d_head=8, seed=seed, window=window,
                         static_bidirectional=bidir)
        do = draw_grad(wl)
        dq, dk, dv = _bwd(wl, do)
        for r in range(wl.num_requests):
            a, b = wl.request(r)
            if b == a:
                continue
            vis = oracle.visibility(wl.seg_kind[a:b], wl.timestamps[a:b], delay=0,
                                    window=window, static_bidirectional=bidir)
            assert vis.any(axis=1).all()
            t = lambda x: torch.from_numpy(np.ascontiguousarray(
                x[a:b].astype(np.float64).transpose(1, 0, 2))).requires_grad_(True)
            tq, tk, tv = t(wl.q), t(wl.k), t(wl.v)
            o = torch.nn.functional.scaled_dot_product_attention(
                tq, tk, tv, attn_mask=torch.from_numpy(vis))
            o.backward(torch.from_numpy(np.ascontiguousarray(
                do[a:b].astype(np.float64).transpose(1, 0, 2))))
            for got, ref in ((dq, tq), (dk, tk), (dv, tv)):
                assert np.allclose(got[a:b], ref.grad.numpy().transpose(1, 0, 2),
                                   atol=1e-12, rtol=0)


def test_backward_matches_finite_differences_with_rope():
    """Central differences of L = sum(dO * O) through the oracle forward, on
    every segment kind, with the delay rule, time RoPE and an empty row."""
    reqs = [[(PROFILE, np.full(2, NOW - 5000, np.int64)),
             (HISTORY, np.array([NOW - 4000, NOW - 3000, NOW - 2900, NOW - 1000])),
             (REALTIME, np.array([NOW - 500, NOW - 200, NOW - 200])),
             (CANDIDATE, np.array([NOW - 300, NOW, NOW - 600]))],
            [(HISTORY, np.array([NOW - 90, NOW - 80, NOW - 10])),
             (CANDIDATE, np.array([NOW]))]]
    for bidir, delay, window in ((False, 60, 0), (True, 0, 0), (False, 0, 2)):
        wl = make_custom(reqs, heads=2, d_head=6, seed=3, delay=delay, window=window,
                         static_bidirectional=bidir)
        do = draw_grad(wl).astype(np.float64)
        q, k, v = (x.astype(np.float64) for x in (wl.q, wl.k, wl.v))
        grads = _bwd(wl, do, rope=ROPE)
        loss = lambda q_, k_, v_: float((_fwd(wl, q_, k_, v_, rope=ROPE) * do).sum())
        rng = np.random.default_rng(delay + window + int(bidir))
        h = 1e-5
        for which in range(3):
            for _ in range(12):
                idx = tuple(int(rng.integers(0, n)) for n in q.shape)
                xs = [q.copy(), k.copy(), v.copy()]
                xs[which][idx] += h
                lp = loss(*xs)
                xs[which][idx] -= 2 * h
                lm = loss(*xs)
                fd = (lp - lm) / (2 * h)
                assert grads[which][idx] == pytest.approx(fd, abs=1e-8, rel=1e-6), (which, idx)


def test_row_that_sees_only_itself():
    """window = 1: every history row sees exactly its own key, so O_i = V_i,
    dV_i = dO_i and dQ_i = dK_i = 0 (up to rounding)."""
    hist = np.arange(NOW - 50, NOW, 1, dtype=np.int64)
    wl = make_custom([[(HISTORY, hist)]], heads=2, d_head=8, seed=4, window=1)
    do = draw_grad(wl)
    dq, dk, dv = _bwd(wl, do, rope=ROPE)
    assert np.allclose(dv, do, atol=1e-14, rtol=0)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13


def test_empty_rows_and_unseen_keys_get_zero_gradients():
    # history only, one-hour delay: the first rows see nothing and the keys of
    # the last hour are seen by no row
    hist = np.sort(np.random.default_rng(7).integers(NOW - 6 * 3600, NOW, size=60))
    wl = make_custom([[(HISTORY, hist)]], heads=2, d_head=8, seed=7, delay=3600)
    do = draw_grad(wl)
    dq, dk, dv = _bwd(wl, do, rope=ROPE)
    vis = oracle.visibility(wl.seg_kind, wl.timestamps, delay=wl.delay, window=0,
                            static_bidirectional=False)
    empty_rows = ~vis.any(axis=1)
    unseen_keys = ~vis.any(axis=0)
    assert empty_rows.sum() >= 1 and unseen_keys.sum() >= 1
    assert np.all(dq[empty_rows] == 0.0)
    assert np.all(dk[unseen_keys] == 0.0) and np.all(dv[unseen_keys] == 0.0)
    # every other row / key gets a non-trivial gradient
    assert np.all(np.abs(dq[~empty_rows]).sum(axis=(1, 2)) > 0)


@pytest.mark.parametrize("cfg_seed", [5, 6])
def test_translation_and_scaling_invariants(cfg_seed):
    rng = np.random.default_rng(cfg_seed)
    reqs = random_layout(rng, 4, 70)
    wl = make_custom(reqs, heads=3, d_head=8, seed=cfg_seed, delay=3600, window=9,
                     global_tail=3)
    do = draw_grad(wl)
    dq, dk, dv = _bwd(wl, do, rope=ROPE)
    o = _fwd(wl, wl.q.astype(np.float64), wl.k.astype(np.float64), wl.v.astype(np.float64),
             rope=ROPE)
    for r in range(wl.num_requests):
        a, b = wl.request(r)
        if b == a:
            continue
        # gradients with respect to the rotated keys sum to zero per head
        gk_rot = oracle.time_rope(dk[a:b], wl.timestamps[a:b], **ROPE)
        assert np.abs(gk_rot.sum(axis=0)).max() < 1e-12
        # sum_j dV_j = sum of dO over rows that see at least one key
        vis = oracle.visibility(wl.seg_kind[a:b], wl.timestamps[a:b], delay=wl.delay,
                                window=wl.window, static_bidirectional=False,
                                global_tail=wl.global_tail)
        has = vis.any(axis=1)
        assert np.allclose(dv[a:b].sum(axis=0), do[a:b][has].astype(np.float64).sum(axis=0),
                           atol=1e-12)
        assert np.all(o[a:b][~has] == 0.0)
        # bilinearity of the scores: sum q.dq == sum k.dk per head
        lhs = (wl.q[a:b].astype(np.float64) * dq[a:b]).sum(axis=(0, 2))
        rhs = (wl.k[a:b].astype(np.float64) * dk[a:b]).sum(axis=(0, 2))
        assert np.allclose(lhs, rhs, atol=1e-11)


def test_time_shift_invariance_of_gradients():
    wl = make_config(1)
    do = draw_grad(wl)
    g0 = _bwd(wl, do, rope=ROPE)
    for shift in (10**9, -NOW, 12_345.678):
        g1 = _bwd(wl, do, rope=ROPE, rope_times=wl.timestamps.astype(np.float64) + shift)
        for x0, x1 in zip(g0, g1):
            assert np.allclose(x0, x1, atol=1e-9, rtol=0)


def test_heads_and_requests_subsets():
    rng = np.random.default_rng(9)
    wl = make_custom(random_layout(rng, 3, 40, allow_empty=False), heads=3, d_head=4, seed=9,
                     delay=60)
    do = draw_grad(wl)
    full = _bwd(wl, do, rope=ROPE)
    part = _bwd(wl, do, rope=ROPE, heads=[1], requests=[0, 2])
    a0, b0 = wl.request(0)
    a2, b2 = wl.request(2)
    a1, b1 = wl.request(1)
    for f, p in zip(full, part):
        assert np.array_equal(p[a0:b0, 1], f[a0:b0, 1])
        assert np.array_equal(p[a2:b2, 1], f[a2:b2, 1])
        assert np.all(p[:, [0, 2]] == 0.0) and np.all(p[a1:b1] == 0.0)


@pytest.mark.parametrize("seed", [11, 12])
def test_sampled_backward_equals_full(seed):
    """The sampled form (row statistics first, sums over row blocks) gives
    the full backward's entries."""
    rng = np.random.default_rng(seed)
    reqs = random_layout(rng, 3, 300, allow_empty=False)
    wl = make_custom(reqs, heads=2, d_head=8, seed=seed, delay=600, window=40, global_tail=5)
    do = draw_grad(wl)
    dq, dk, dv = _bwd(wl, do, rope=ROPE)
    for r in range(wl.num_requests):
        a, b = wl.request(r)
        rows = rng.choice(b - a, size=min(9, b - a), replace=False)
        keys = rng.choice(b - a, size=min(7, b - a), replace=False)
        for h in range(2):
            sq, sk_, sv = oracle.attention_backward_sampled(
                wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q, wl.k, wl.v, do, request=r,
                head=h, rows=rows, keys=keys, delay=wl.delay, window=wl.window,
                static_bidirectional=False, rope=ROPE, global_tail=wl.global_tail, row_block=37)
            assert np.allclose(sq, dq[a + rows, h], atol=1e-12, rtol=0)
            assert np.allclose(sk_, dk[a + keys, h], atol=1e-12, rtol=0)
            assert np.allclose(sv, dv[a + keys, h], atol=1e-12, rtol=0)
