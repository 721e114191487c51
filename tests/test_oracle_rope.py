"""Pins for the oracle's time RoPE (CPU only): closed forms at d = 2, the CADET
page's worked constants, norm preservation and time-shift invariance of
rotated dot products."""

import json
import math
import os

import numpy as np
import pytest

import oracle
from rk_workloads import BASE, DT_MAX, NOW, PHI_MIN, YEAR

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DAY = 86400.0


def _g():
    with open(os.path.join(GOLDEN, "cadet_rope_constants.json")) as f:
        return json.load(f)


def test_d2_closed_form_slowest_pair_turns_phi_min_per_window():
    """At d = 2 there is one pair with omega_0 = phi_min / dt_max: over one full
    look-back window (1 yr) it turns exactly phi_min radians."""
    x = np.array([[1.0, 0.0]])
    out = oracle.time_rope(x, np.array([DT_MAX]), phi_min=PHI_MIN, dt_max=DT_MAX, base=BASE)
    assert out[0, 0] == pytest.approx(math.cos(1e-4), abs=1e-15)
    assert out[0, 1] == pytest.approx(math.sin(1e-4), abs=1e-15)
    # counter-clockwise on (x0, x1) = (0, 1) as well
    out = oracle.time_rope(np.array([[0.0, 1.0]]), np.array([DT_MAX]), phi_min=PHI_MIN,
                           dt_max=DT_MAX, base=BASE)
    assert out[0, 0] == pytest.approx(-math.sin(1e-4), abs=1e-15)
    assert out[0, 1] == pytest.approx(math.cos(1e-4), abs=1e-15)


def test_frequencies_grow_with_pair_index_as_printed():
    """omega_i = phi_min/dt_max * base^(2i/d): ratio between consecutive pairs
    is base^(2/d), first pair phi_min/dt_max."""
    for d in (2, 4, 32, 64):
        w = oracle.rope_frequencies(d, PHI_MIN, DT_MAX, BASE)
        assert w.shape == (d // 2,)
        assert w[0] == pytest.approx(PHI_MIN / DT_MAX, rel=1e-15)
        if d > 2:
            assert np.allclose(w[1:] / w[:-1], BASE ** (2.0 / d), rtol=1e-13)


def test_page_worked_constants():
    g = _g()
    # fastest hand per the page's approximation: phi_min * base rad per year
    fastest = g["phi_min"] * g["base"]
    assert fastest == pytest.approx(g["fastest_rad_per_year"], rel=1e-12)
    assert 2 * math.pi / fastest * g["year_days"] == pytest.approx(g["full_turn_days"], abs=0.05)
    assert fastest / g["year_days"] == pytest.approx(g["rad_per_day"], abs=0.005)
    assert fastest / (g["year_days"] * 24) == pytest.approx(g["rad_per_hour"], abs=0.0005)
    # the oracle's highest pair approaches that hand from below as d grows
    w = oracle.rope_frequencies(1024, PHI_MIN, DT_MAX, BASE)
    assert w[-1] * DT_MAX < fastest
    assert w[-1] * DT_MAX == pytest.approx(fastest, rel=0.03)


@pytest.mark.parametrize("rad_per_year,key", [("fastest_rad_per_year", "readout_fastest"),
                                               ("slower_rad_per_year", "readout_slower")])
def test_page_readout_38_days(rad_per_year, key):
    """Rotate the same unit vector at two times 38 days apart with a single
    pair turning `rad_per_year`; the dot product is the page's readout."""
    g = _g()
    speed = g[rad_per_year]
    # one pair (d = 2) whose omega_0 = phi_min/dt_max equals `speed` per year
    kw = dict(phi_min=speed, dt_max=g["year_days"] * DAY, base=BASE)
    t1 = np.array([0.0])
    t2 = np.array([g["readout_days"] * DAY])
    q = oracle.time_rope(np.array([[1.0, 0.0]]), t2, **kw)
    k = oracle.time_rope(np.array([[1.0, 0.0]]), t1, **kw)
    assert round(float(q[0] @ k[0]), 2) == pytest.approx(g[key], abs=1e-12)


def test_rotation_preserves_norm():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 3, 64))
    t = rng.integers(NOW - YEAR, NOW, size=50)
    y = oracle.time_rope(x, t, phi_min=PHI_MIN, dt_max=DT_MAX, base=BASE)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def test_dot_products_depend_only_on_time_difference():
    """CADET: attention between two events depends only on their time
    difference.  Shift every time by the same amount (also by amounts that
    are not whole periods of any pair) -> q.k unchanged."""
    rng = np.random.default_rng(1)
    q = rng.standard_normal((40, 64))
    k = rng.standard_normal((40, 64))
    t = rng.integers(NOW - YEAR, NOW, size=40)
    kw = dict(phi_min=PHI_MIN, dt_max=DT_MAX, base=BASE)
    s0 = oracle.time_rope(q, t, **kw) @ oracle.time_rope(k, t, **kw).T
    for shift in (-NOW, 1_000_000_000, 12_345.678):
        ts = t + shift
        s1 = oracle.time_rope(q, ts, **kw) @ oracle.time_rope(k, ts, **kw).T
        assert np.allclose(s0, s1, atol=1e-9)
    # and it does change with the time difference
    s2 = oracle.time_rope(q, t, **kw) @ oracle.time_rope(k, t + 86400 * 30, **kw).T
    assert not np.allclose(s0, s2, atol=1e-3)


def test_zero_time_is_identity():
    x = np.random.default_rng(2).standard_normal((5, 2, 32))
    y = oracle.time_rope(x, np.zeros(5), phi_min=PHI_MIN, dt_max=DT_MAX, base=BASE)
    assert np.array_equal(x, y)
