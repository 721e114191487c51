"""LazFormer layout functions of the C ABI (host code, no GPU) against the
oracle's compression and pruning: output layouts (offsets, kinds,
timestamps) equal, and the row ranges reproduce the oracle's rows when
applied to the input on the CPU; eq. 22 lengths equal the oracle's; host
validation errors."""

import ctypes as C

import numpy as np
import pytest

import oracle
from rk_workloads import HISTORY, NOW, PROFILE, REALTIME, make_custom, random_layout


@pytest.fixture(scope="module")
def rk():
    import masked_attention_amd as m
    from masked_attention_amd import _rk
    _rk.lib()
    return m


def _apply(ranges, x):
    return np.stack([x[b:e].sum(axis=0) for b, e in ranges]) if len(ranges) else x[:0]


@pytest.mark.parametrize("seed", range(4))
def test_compress_layout_matches_oracle(rk, seed):
    rng = np.random.default_rng(seed)
    wl = make_custom(random_layout(rng, 7, 400), heads=1, d_head=2, seed=seed, with_qkv=False)
    x = rng.standard_normal((wl.total_tokens, 3))
    lay = rk.Layout.from_workload(wl)
    for keep, group in ((0, 4), (256, 8), (30, 16), (10 ** 6, 2), (5, 1)):
        out = rk.rk_compress_layout(lay, keep=keep, group=group)
        offs, kinds, times, y = oracle.group_sum_compress(wl.req_offsets, wl.seg_kind,
                                                          wl.timestamps, x, keep=keep,
                                                          group=group)
        assert np.array_equal(out.req_offsets, offs)
        assert np.array_equal(out.seg_kind, kinds)
        assert np.array_equal(out.timestamps, times)
        assert np.allclose(_apply(out.ranges, x), y, atol=1e-12)


def test_compress_length_table(rk):
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "lazformer_lengths.json")))
    L = g["history_length"]
    wl = make_custom([[(HISTORY, np.arange(NOW - L, NOW, dtype=np.int64))]], heads=1, d_head=2,
                     seed=0, with_qkv=False)
    for row in g["compression_table"]:
        out = rk.rk_compress_layout(rk.Layout.from_workload(wl), keep=row["keep"],
                                    group=row["group"])
        assert out.T == row["length"]


def test_pruned_lengths_match_oracle(rk):
    for l_tilde in (0, 1, 100, 129, 131, 1152, 5000):
        for n_layers in (1, 2, 3, 5, 12):
            for layer in range(1, n_layers + 1):
                assert rk.rk_pruned_history_length(l_tilde, 128, layer, n_layers) == \
                    oracle.pruned_history_length(l_tilde, 128, layer, n_layers)
    assert [rk.rk_pruned_history_length(1152, 128, l, 5) for l in range(1, 6)] == \
        [1152, 896, 640, 384, 128]


@pytest.mark.parametrize("seed", range(3))
def test_prune_layout_matches_oracle(rk, seed):
    rng = np.random.default_rng(10 + seed)
    wl = make_custom(random_layout(rng, 6, 500), heads=1, d_head=2, seed=seed, with_qkv=False)
    x = rng.standard_normal((wl.total_tokens, 2))
    lay = rk.Layout.from_workload(wl)
    lt = lay.history_lengths()
    for layer in range(1, 5):
        out = rk.rk_prune_layout(lay, l_tilde=lt, n_min=8, layer=layer, num_layers=4)
        offs, kinds, times, y = oracle.prune_history(wl.req_offsets, wl.seg_kind, wl.timestamps,
                                                     x, l_tilde=lt, n_min=8, layer=layer,
                                                     num_layers=4)
        assert np.array_equal(out.req_offsets, offs)
        assert np.array_equal(out.seg_kind, kinds)
        assert np.array_equal(out.timestamps, times)
        assert np.array_equal(_apply(out.ranges, x), y)


def test_layout_host_errors(rk):
    from masked_attention_amd import _rk
    lib = _rk.lib()
    wl = make_custom([[(HISTORY, np.array([NOW - 5, NOW - 9, NOW], np.int64))]], heads=1,
                     d_head=2, seed=0, with_qkv=False)
    lay = rk.Layout.from_workload(wl)
    with pytest.raises(_rk.RkError) as e:
        rk.rk_compress_layout(lay, keep=1, group=2)
    assert e.value.status == _rk.RK_ERR_UNSORTED_TIME
    bad = rk.Layout(wl.req_offsets, np.array([1, 0, 1], np.uint8), np.array([1, 2, 3]))
    with pytest.raises(_rk.RkError) as e:
        rk.rk_compress_layout(bad, keep=1, group=2)
    assert e.value.status == _rk.RK_ERR_SEGMENT_ORDER
    good = rk.Layout(wl.req_offsets, wl.seg_kind, np.sort(wl.timestamps))
    for keep, group in ((-1, 2), (1, 0)):
        with pytest.raises(_rk.RkError) as e:
            rk.rk_compress_layout(good, keep=keep, group=group)
        assert e.value.status == _rk.RK_ERR_INVALID_ARG
    n = C.c_int32()
    for args in ((10, 1, 0, 3), (10, 1, 4, 3), (-1, 1, 1, 1), (10, 1, 1, 0)):
        assert lib.rk_pruned_history_length(*args, C.byref(n)) == _rk.RK_ERR_INVALID_ARG
    assert lib.rk_compress_layout(None, 1, 1, None) == _rk.RK_ERR_INVALID_ARG
    assert lib.rk_gather_sum(None, 4, 4, None, 1, None, 1, 1, 7, None) == _rk.RK_ERR_INVALID_ARG
    assert lib.rk_gather_sum(None, -1, 4, None, 1, None, 1, 1, 0, None) == _rk.RK_ERR_INVALID_ARG
