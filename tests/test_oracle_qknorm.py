"""Pins for the oracle's QK Norm (CPU only): the RMSNorm of every [d] row of
Q and K before the rotation (TM20K section 2; SORT section 3.3.2).

* torch.nn.functional.rms_norm in float64 (a library routine) gives the
  same rows, with and without a gain;
* with gain 1 every row has unit root-mean-square (up to eps);
* rows are scale invariant (norm(c x) = norm(x), c > 0, up to eps);
* attention with qk_norm equals attention on inputs normalised beforehand.
"""

import numpy as np
import torch

import oracle
from rk_workloads import make_custom, random_layout

ROPE = dict(phi_min=1e-4, dt_max=31_536_000.0, base=6e5)


def test_matches_torch_rms_norm():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 3, 64)) * rng.uniform(0.1, 10, size=(50, 3, 1))
    g = rng.uniform(0.5, 2.0, size=64)
    for gamma in (None, g):
        ref = torch.nn.functional.rms_norm(
            torch.from_numpy(x), (64,), weight=None if gamma is None else torch.from_numpy(gamma),
            eps=1e-6).numpy()
        assert np.allclose(oracle.qk_rmsnorm(x, gamma, 1e-6), ref, atol=1e-13, rtol=1e-12)


def test_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((40, 32)) * 5.0
    y = oracle.qk_rmsnorm(x, None, 1e-12)
    assert np.allclose(np.sqrt((y * y).mean(axis=-1)), 1.0, atol=1e-10)
    assert np.allclose(oracle.qk_rmsnorm(7.5 * x, None, 1e-12), y, atol=1e-10)


def test_attention_with_qk_norm_equals_prenormalised_inputs():
    rng = np.random.default_rng(2)
    wl = make_custom(random_layout(rng, 3, 80), heads=2, d_head=16, seed=3, delay=600, window=7)
    gq, gk = rng.uniform(0.5, 1.5, 16), rng.uniform(0.5, 1.5, 16)
    margs = dict(delay=wl.delay, window=wl.window, static_bidirectional=False, rope=ROPE)
    o1, l1 = oracle.attention_forward(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q, wl.k,
                                      wl.v, qk_norm=dict(eps=1e-6, gamma_q=gq, gamma_k=gk),
                                      **margs)
    qn = oracle.qk_rmsnorm(wl.q, gq, 1e-6)
    kn = oracle.qk_rmsnorm(wl.k, gk, 1e-6)
    o2, l2 = oracle.attention_forward(wl.req_offsets, wl.seg_kind, wl.timestamps, qn, kn, wl.v,
                                      **margs)
    assert np.array_equal(o1, o2)
    fin = np.isfinite(l2)
    assert np.array_equal(l1[fin], l2[fin])
