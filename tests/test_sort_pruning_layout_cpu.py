"""SORT query-pruning layout functions of the C ABI (host code, no GPU)
against the oracle (SORT, section 3.2.2): the exponential schedule's
lengths, the pruned and pooled layouts (offsets, kinds, timestamps), and the
row ranges, which reproduce the oracle's rows when averaged on the CPU;
the linear schedule through the extended call equals eq. 22; host errors."""

import numpy as np
import pytest

import oracle
from rk_workloads import HISTORY, NOW, make_custom, random_layout


@pytest.fixture(scope="module")
def rk():
    import masked_attention_amd as m
    from masked_attention_amd import _rk
    _rk.lib()
    return m


def _mean(ranges, x):
    rows = [x[b:e].mean(axis=0) if e > b else np.zeros(x.shape[1:]) for b, e in ranges]
    return np.stack(rows) if rows else x[:0]


def test_exp_lengths_match_oracle(rk):
    for l_tilde in (0, 1, 5, 100, 1024, 1152, 5000):
        for decay in (0.3, 0.5, 0.75, 1.0):
            for layer in range(1, 8):
                for n_min in (0, 16, 128):
                    assert rk.rk_pruned_history_length_ex(
                        l_tilde, schedule="exp", n_min=n_min, layer=layer, decay=decay) == \
                        oracle.pruned_history_length_exp(l_tilde, n_min, decay, layer)
    # the linear schedule through the extended call is eq. 22
    assert [rk.rk_pruned_history_length_ex(1152, schedule="linear", n_min=128, layer=l,
                                           num_layers=5) for l in range(1, 6)] == \
        [1152, 896, 640, 384, 128]


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("schedule", ["linear", "exp"])
@pytest.mark.parametrize("pool", [False, True])
def test_prune_layout_ex_matches_oracle(rk, seed, schedule, pool):
    rng = np.random.default_rng(40 + seed)
    wl = make_custom(random_layout(rng, 6, 500), heads=1, d_head=2, seed=seed, with_qkv=False)
    x = rng.standard_normal((wl.total_tokens, 3))
    lay = rk.Layout.from_workload(wl)
    lt = lay.history_lengths()
    for layer in range(1, 5):
        kw = dict(schedule=schedule, n_min=8, layer=layer, num_layers=4, decay=0.6, pool=pool)
        out = rk.rk_prune_layout_ex(lay, l_tilde=lt, **kw)
        if schedule == "linear":
            keep = [oracle.pruned_history_length(int(l), 8, layer, 4) for l in lt]
        else:
            keep = [oracle.pruned_history_length_exp(int(l), 8, 0.6, layer) for l in lt]
        if pool:
            offs, kinds, times, y = oracle.prune_history_pooled(
                wl.req_offsets, wl.seg_kind, wl.timestamps, x, keep=keep)
        else:
            offs, kinds, times, y = oracle.prune_history_keep(
                wl.req_offsets, wl.seg_kind, wl.timestamps, x, keep=keep)
        assert np.array_equal(out.req_offsets, offs)
        assert np.array_equal(out.seg_kind, kinds)
        assert np.array_equal(out.timestamps, times)
        assert np.allclose(_mean(out.ranges, x), y, atol=1e-12)


def test_linear_unpooled_equals_eq22_layout(rk):
    rng = np.random.default_rng(77)
    wl = make_custom(random_layout(rng, 5, 400), heads=1, d_head=2, seed=1, with_qkv=False)
    lay = rk.Layout.from_workload(wl)
    lt = lay.history_lengths()
    for layer in (1, 2, 3):
        a = rk.rk_prune_layout(lay, l_tilde=lt, n_min=4, layer=layer, num_layers=3)
        b = rk.rk_prune_layout_ex(lay, l_tilde=lt, schedule="linear", n_min=4, layer=layer,
                                  num_layers=3)
        for f in ("req_offsets", "seg_kind", "timestamps", "ranges"):
            assert np.array_equal(getattr(a, f), getattr(b, f))


def test_prune_ex_host_errors(rk):
    from masked_attention_amd import _rk
    wl = make_custom([[(HISTORY, np.array([NOW - 9, NOW - 5, NOW], np.int64))]], heads=1,
                     d_head=2, seed=0, with_qkv=False)
    lay = rk.Layout.from_workload(wl)
    for bad in (dict(schedule="exp", n_min=0, layer=1, decay=0.0),
                dict(schedule="exp", n_min=0, layer=1, decay=1.5),
                dict(schedule="exp", n_min=-1, layer=1, decay=0.5),
                dict(schedule="exp", n_min=0, layer=0, decay=0.5),
                dict(schedule="linear", n_min=0, layer=3, num_layers=2)):
        with pytest.raises(_rk.RkError) as e:
            rk.rk_prune_layout_ex(lay, l_tilde=[3], **bad)
        assert e.value.status == _rk.RK_ERR_INVALID_ARG
        with pytest.raises(_rk.RkError):
            rk.rk_pruned_history_length_ex(3, **bad)
