"""Pins of the oracle's SORT query-pruning functions (SORT, section 3.2.2):
the exponential schedule and the pooled form.  The page names the
strategies without formulas; the oracle follows the reading stated in its
header, and these tests pin it to that reading's mathematics: closed forms
of the schedule, the identity cases, conservation of each request's history
total under pooling, and a hand-built brute-force case."""

import numpy as np
import pytest

import oracle
from oracle import CANDIDATE, HISTORY, PROFILE, REALTIME


def test_exp_schedule_closed_forms():
    # halving from 1024: 1024, 512, 256, 128, 64
    assert [oracle.pruned_history_length_exp(1024, 0, 0.5, l) for l in range(1, 6)] == \
        [1024, 512, 256, 128, 64]
    # the floor N_min stops the decay
    assert [oracle.pruned_history_length_exp(1024, 100, 0.5, l) for l in range(1, 7)] == \
        [1024, 512, 256, 128, 100, 100]
    # 1000 * 0.3^(l-1): 1000, 300, 90, 27 (27.0 exactly), 8.1 -> 8
    assert [oracle.pruned_history_length_exp(1000, 0, 0.3, l) for l in range(1, 6)] == \
        [1000, 300, 90, 27, 8]
    # halves round away from zero: 5 * 0.5 = 2.5 -> 3; 7 * 0.5 = 3.5 -> 4
    assert oracle.pruned_history_length_exp(5, 0, 0.5, 2) == 3
    assert oracle.pruned_history_length_exp(7, 0, 0.5, 2) == 4


@pytest.mark.parametrize("l_tilde", [0, 1, 37, 1152])
def test_exp_schedule_identities(l_tilde):
    for layer in range(1, 8):
        # decay 1 keeps everything; the first layer always keeps L~
        assert oracle.pruned_history_length_exp(l_tilde, 0, 1.0, layer) == l_tilde
    for decay in (0.1, 0.5, 0.9):
        assert oracle.pruned_history_length_exp(l_tilde, 0, decay, 1) == l_tilde
        seq = [oracle.pruned_history_length_exp(l_tilde, 16, decay, l) for l in range(1, 12)]
        assert all(a >= b for a, b in zip(seq, seq[1:]))          # non-increasing
        assert all(min(l_tilde, 16) <= n <= l_tilde for n in seq)  # floor and cap


def _layout(rng, R, max_len):
    offs, kinds, times = [0], [], []
    for _ in range(R):
        n = [int(v) for v in rng.integers(0, max_len, 4)]
        for kd, c in zip((PROFILE, HISTORY, REALTIME, CANDIDATE), n):
            kinds += [kd] * c
            t0 = int(rng.integers(10**6, 2 * 10**6))
            times += list(np.sort(rng.integers(t0, t0 + 10**5, c))) if kd == HISTORY else \
                [int(v) for v in rng.integers(0, 10**6, c)]
        offs.append(offs[-1] + sum(n))
    return np.asarray(offs, np.int32), np.asarray(kinds, np.uint8), np.asarray(times, np.int64)


@pytest.mark.parametrize("seed", range(4))
def test_pooled_conserves_history_total(seed):
    rng = np.random.default_rng(seed)
    offs, kinds, times = _layout(rng, 6, 40)
    x = rng.standard_normal((kinds.shape[0], 3))
    R = offs.shape[0] - 1
    n_hist = np.array([int((kinds[offs[r]:offs[r + 1]] == HISTORY).sum()) for r in range(R)])
    keep = rng.integers(0, 45, R)
    o2, k2, t2, y = oracle.prune_history_pooled(offs, kinds, times, x, keep=keep)
    for r in range(R):
        a, b = offs[r], offs[r + 1]
        a2, b2 = o2[r], o2[r + 1]
        dropped = max(0, n_hist[r] - keep[r])
        # one pooled token replaces the dropped ones
        assert b2 - a2 == (b - a) - dropped + (1 if dropped else 0)
        # pooled mean times its count plus the kept history = the history total
        hist_in = x[a:b][kinds[a:b] == HISTORY]
        hist_out = y[a2:b2][k2[a2:b2] == HISTORY]
        if dropped:
            total = hist_out[0] * dropped + hist_out[1:].sum(axis=0)
        else:
            total = hist_out.sum(axis=0)
        assert np.allclose(total, hist_in.sum(axis=0), atol=1e-12)
        # non-history tokens pass through unchanged, in order
        assert np.array_equal(k2[a2:b2][k2[a2:b2] != HISTORY], kinds[a:b][kinds[a:b] != HISTORY])
        assert np.array_equal(y[a2:b2][k2[a2:b2] != HISTORY], x[a:b][kinds[a:b] != HISTORY])


def test_pooled_by_hand():
    # one request: P, H1..H5 at times 10..50, R, C; keep the last 2 history tokens
    kinds = np.array([PROFILE, HISTORY, HISTORY, HISTORY, HISTORY, HISTORY, REALTIME, CANDIDATE],
                     np.uint8)
    times = np.array([5, 10, 20, 30, 40, 50, 55, 60], np.int64)
    x = np.arange(8, dtype=np.float64)[:, None] * np.array([[1.0, -2.0]])
    o2, k2, t2, y = oracle.prune_history_pooled(np.array([0, 8], np.int32), kinds, times, x,
                                                keep=[2])
    assert list(o2) == [0, 6]
    assert list(k2) == [PROFILE, HISTORY, HISTORY, HISTORY, REALTIME, CANDIDATE]
    assert list(t2) == [5, 30, 40, 50, 55, 60]  # the pooled token carries H3's time
    assert np.allclose(y[1], [2.0, -4.0])      # mean of rows 1, 2, 3
    assert np.allclose(y[[0, 2, 3, 4, 5]], x[[0, 4, 5, 6, 7]])
    # keeping everything (or more) is the identity
    o3, k3, t3, y3 = oracle.prune_history_pooled(np.array([0, 8], np.int32), kinds, times, x,
                                                 keep=[5])
    assert np.array_equal(k3, kinds) and np.array_equal(t3, times) and np.allclose(y3, x)
    # keeping nothing pools the whole history into one token
    o4, k4, t4, y4 = oracle.prune_history_pooled(np.array([0, 8], np.int32), kinds, times, x,
                                                 keep=[0])
    assert list(k4) == [PROFILE, HISTORY, REALTIME, CANDIDATE] and t4[1] == 50
    assert np.allclose(y4[1], x[1:6].mean(axis=0))


@pytest.mark.parametrize("seed", range(3))
def test_keep_form_matches_eq22_pruning(seed):
    """Pruning to given lengths reduces to the eq. 22 pruning when the
    lengths come from eq. 22, and pooling with nothing dropped to it too."""
    rng = np.random.default_rng(60 + seed)
    offs, kinds, times = _layout(rng, 5, 30)
    x = rng.standard_normal((kinds.shape[0], 2))
    R = offs.shape[0] - 1
    lt = np.array([int((kinds[offs[r]:offs[r + 1]] == HISTORY).sum()) for r in range(R)])
    for layer in (1, 2, 3):
        keep = [oracle.pruned_history_length(int(l), 3, layer, 3) for l in lt]
        a = oracle.prune_history(offs, kinds, times, x, l_tilde=lt, n_min=3, layer=layer,
                                 num_layers=3)
        b = oracle.prune_history_keep(offs, kinds, times, x, keep=keep)
        for u, v in zip(a, b):
            assert np.array_equal(u, v)
    c = oracle.prune_history_pooled(offs, kinds, times, x, keep=lt)
    d = oracle.prune_history_keep(offs, kinds, times, x, keep=lt)
    for u, v in zip(c, d):
        assert np.allclose(u, v)
