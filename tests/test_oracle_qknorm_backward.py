"""Pins for the oracle's backward through QK Norm (CPU only): gradients of
the attention forward whose Q and K rows are RMS-normalised (with gains)
before the rotation (TM20K section 2; SORT section 3.3.2), taken back
through the norm by the chain rule.

* qk_rmsnorm_backward equals torch autograd of torch's own rms_norm in
  float64 (a library routine), with and without a gain, for dx and dgain;
* at eps = 0 the norm is scale invariant, so every row's gradient is
  orthogonal to the row (sum_j x_j dx_j = 0);
* attention_backward_qk_norm equals torch autograd of the whole forward
  (rms_norm, scaled scores, explicit mask, softmax, P V) without RoPE;
* with RoPE, central finite differences of sum(dO * O) through the oracle
  forward (attention_forward with qk_norm) match dq, dk and both gains'
  gradients at sampled coordinates;
* with gains 1 and no gain the gradients of q, k, v agree (the gain only
  scales).
"""

import numpy as np
import torch

import oracle
from rk_workloads import make_custom, random_layout

ROPE = dict(phi_min=1e-4, dt_max=31_536_000.0, base=6e5)


def test_norm_backward_matches_torch_autograd():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((30, 2, 16)) * rng.uniform(0.2, 5.0, size=(30, 2, 1))
    g = rng.standard_normal((30, 2, 16))
    gam = rng.uniform(0.5, 2.0, 16)
    for gamma in (None, gam):
        xt = torch.from_numpy(x).requires_grad_(True)
        wt = None if gamma is None else torch.from_numpy(gamma).requires_grad_(True)
        y = torch.nn.functional.rms_norm(xt, (16,), weight=wt, eps=1e-5)
        (y * torch.from_numpy(g)).sum().backward()
        dx, dgam = oracle.qk_rmsnorm_backward(x, gamma, 1e-5, g)
        assert np.allclose(dx, xt.grad.numpy(), atol=1e-12, rtol=1e-11)
        if gamma is None:
            assert dgam is None
        else:
            assert np.allclose(dgam, wt.grad.numpy(), atol=1e-11, rtol=1e-11)


def test_gradient_orthogonal_to_row_at_zero_eps():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((40, 32)) * 3.0
    g = rng.standard_normal((40, 32))
    dx, _ = oracle.qk_rmsnorm_backward(x, rng.uniform(0.5, 1.5, 32), 0.0, g)
    assert np.abs((x * dx).sum(axis=-1)).max() < 1e-11 * np.abs(dx).max() * np.abs(x).max() * 32


def _torch_forward(wl, q, k, v, gq, gk, eps, scale):
    """The forward with torch ops (no RoPE): rms_norm, scores, explicit mask,
    softmax (rows with no visible key give 0), P V."""
    outs = []
    for r in range(wl.num_requests):
        a, b = wl.request(r)
        if b == a:
            continue
        vis = torch.from_numpy(oracle.visibility(wl.seg_kind[a:b], wl.timestamps[a:b],
                                                 delay=wl.delay, window=wl.window,
                                                 static_bidirectional=wl.static_bidirectional))
        qn = torch.nn.functional.rms_norm(q[a:b], (q.shape[-1],), weight=gq, eps=eps)
        kn = torch.nn.functional.rms_norm(k[a:b], (k.shape[-1],), weight=gk, eps=eps)
        for h in range(q.shape[1]):
            s = (qn[:, h] @ kn[:, h].T.contiguous()) * scale
            s = s.masked_fill(~vis, float("-inf"))
            has = vis.any(dim=1, keepdim=True)
            p = torch.softmax(torch.where(has, s, torch.zeros_like(s)), dim=1) * has
            p = torch.where(vis, p, torch.zeros_like(p))
            outs.append((a, b, h, p @ v[a:b, h]))
    return outs


def test_attention_qk_norm_backward_matches_autograd():
    rng = np.random.default_rng(2)
    wl = make_custom(random_layout(rng, 3, 70), heads=2, d_head=16, seed=5, delay=600, window=9)
    gq, gk = rng.uniform(0.5, 1.5, 16), rng.uniform(0.5, 1.5, 16)
    do = rng.standard_normal(wl.q.shape)
    eps, scale = 1e-6, 0.3
    q = torch.from_numpy(wl.q.astype(np.float64)).requires_grad_(True)
    k = torch.from_numpy(wl.k.astype(np.float64)).requires_grad_(True)
    v = torch.from_numpy(wl.v.astype(np.float64)).requires_grad_(True)
    tq = torch.from_numpy(gq).requires_grad_(True)
    tk = torch.from_numpy(gk).requires_grad_(True)
    loss = 0.0
    for a, b, h, o in _torch_forward(wl, q, k, v, tq, tk, eps, scale):
        loss = loss + (o * torch.from_numpy(do[a:b, h])).sum()
    loss.backward()
    dq, dk, dv, dgq, dgk = oracle.attention_backward_qk_norm(
        wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q, wl.k, wl.v, do,
        qk_norm=dict(eps=eps, gamma_q=gq, gamma_k=gk), delay=wl.delay, window=wl.window,
        static_bidirectional=False, scale=scale)
    for got, ref in ((dq, q.grad), (dk, k.grad), (dv, v.grad), (dgq, tq.grad), (dgk, tk.grad)):
        assert np.allclose(got, ref.numpy(), atol=1e-10, rtol=1e-9)


def test_attention_qk_norm_backward_finite_differences_with_rope():
    rng = np.random.default_rng(3)
    wl = make_custom(random_layout(rng, 2, 40), heads=1, d_head=8, seed=7, delay=0, window=0)
    gq, gk = rng.uniform(0.5, 1.5, 8), rng.uniform(0.5, 1.5, 8)
    do = rng.standard_normal(wl.q.shape)
    eps = 1e-6
    margs = dict(delay=0, window=0, static_bidirectional=False, rope=ROPE)
    q, k, v = (x.astype(np.float64) for x in (wl.q, wl.k, wl.v))

    def loss(q_, k_, gq_, gk_):
        o, _ = oracle.attention_forward(wl.req_offsets, wl.seg_kind, wl.timestamps, q_, k_, v,
                                        qk_norm=dict(eps=eps, gamma_q=gq_, gamma_k=gk_), **margs)
        return float((o * do).sum())

    dq, dk, _, dgq, dgk = oracle.attention_backward_qk_norm(
        wl.req_offsets, wl.seg_kind, wl.timestamps, q, k, v, do,
        qk_norm=dict(eps=eps, gamma_q=gq, gamma_k=gk), **margs)
    h = 1e-6
    for _ in range(6):
        t, c = int(rng.integers(wl.total_tokens)), int(rng.integers(8))
        for arr, grad, which in ((q, dq, "q"), (k, dk, "k")):
            p, m = arr.copy(), arr.copy()
            p[t, 0, c] += h
            m[t, 0, c] -= h
            fd = (loss(p, k, gq, gk) - loss(m, k, gq, gk) if which == "q"
                  else loss(q, p, gq, gk) - loss(q, m, gq, gk)) / (2 * h)
            assert abs(fd - grad[t, 0, c]) <= 1e-6 * max(1.0, abs(fd)), (which, t, c)
    for c in range(8):
        e = np.zeros(8)
        e[c] = h
        fdq = (loss(q, k, gq + e, gk) - loss(q, k, gq - e, gk)) / (2 * h)
        fdk = (loss(q, k, gq, gk + e) - loss(q, k, gq, gk - e)) / (2 * h)
        assert abs(fdq - dgq[c]) <= 1e-6 * max(1.0, abs(fdq))
        assert abs(fdk - dgk[c]) <= 1e-6 * max(1.0, abs(fdk))


def test_unit_gains_match_no_gain():
    rng = np.random.default_rng(4)
    wl = make_custom(random_layout(rng, 2, 50), heads=2, d_head=16, seed=9, delay=0, window=0)
    do = rng.standard_normal(wl.q.shape)
    kw = dict(delay=0, window=0, static_bidirectional=False, rope=ROPE)
    a = oracle.attention_backward_qk_norm(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q, wl.k,
                                          wl.v, do, qk_norm=dict(eps=1e-6), **kw)
    b = oracle.attention_backward_qk_norm(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q, wl.k,
                                          wl.v, do,
                                          qk_norm=dict(eps=1e-6, gamma_q=np.ones(16),
                                                       gamma_k=np.ones(16)), **kw)
    for x, y in zip(a[:3], b[:3]):
        assert np.allclose(x, y, atol=1e-13, rtol=1e-12)
    assert a[3] is None and a[4] is None and b[3].shape == (16,)
