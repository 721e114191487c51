"""Pins for the oracle's 128 x 64 tile plan (CPU only): closed-form tile
counts of a causal request, class definitions, CSR order and the total."""

import numpy as np
import pytest

import oracle
from rk_workloads import CANDIDATE, HISTORY, NOW, make_config, make_custom, random_layout


def test_causal_tiles_closed_form():
    L = 512
    seg = np.full(L, HISTORY, np.uint8)
    ts = np.arange(L, dtype=np.int64) + NOW
    cnt, cls = oracle.tile_plan_request(seg, ts, delay=0, window=0, static_bidirectional=False)
    assert cnt.shape == (4, 8)
    for qt in range(4):
        for kt in range(8):
            if kt < 2 * qt:
                assert cls[qt, kt] == oracle.FULL and cnt[qt, kt] == 128 * 64
            elif kt == 2 * qt:
                # sum_{r=0}^{127} min(r+1, 64) = 2080 + 64*64
                assert cls[qt, kt] == oracle.PARTIAL and cnt[qt, kt] == 6176
            elif kt == 2 * qt + 1:
                # sum_{r=64}^{127} (r-63) = 2080
                assert cls[qt, kt] == oracle.PARTIAL and cnt[qt, kt] == 2080
            else:
                assert cls[qt, kt] == oracle.EMPTY and cnt[qt, kt] == 0
    assert cnt.sum() == L * (L + 1) // 2


def test_ragged_tiles_never_full():
    L = 200  # 2 q-tiles (128 + 72 rows), 4 k-tiles (64 x 3 + 8 cols)
    seg = np.array([HISTORY] * 150 + [CANDIDATE] * 50, np.uint8)
    ts = np.arange(L, dtype=np.int64) + NOW
    cnt, cls = oracle.tile_plan_request(seg, ts, delay=0, window=0, static_bidirectional=True)
    assert cls[1].tolist().count(oracle.FULL) == 0
    assert cls[:, 3].tolist().count(oracle.FULL) == 0
    # bidirectional static: first q-tile, first two k-tiles entirely static -> FULL
    assert cls[0, 0] == oracle.FULL and cls[0, 1] == oracle.FULL
    vis = oracle.visibility(seg, ts, delay=0, window=0, static_bidirectional=True)
    assert cnt.sum() == vis.sum()


@pytest.mark.parametrize("seed", [0, 1])
def test_plan_totals_and_csr(seed):
    rng = np.random.default_rng(seed)
    reqs = random_layout(rng, 5, 400)
    for bidir, delay, window in ((True, 0, 0), (False, 3600, 0), (False, 0, 70)):
        wl = make_custom(reqs, heads=1, d_head=8, with_qkv=False, delay=delay, window=window,
                         static_bidirectional=bidir)
        plan = oracle.tile_plan(wl.req_offsets, wl.seg_kind, wl.timestamps, delay=delay,
                                window=window, static_bidirectional=bidir)
        total = 0
        off = 0
        q = 0
        for r in range(wl.num_requests):
            a, b = wl.request(r)
            L = b - a
            vis = oracle.visibility(wl.seg_kind[a:b], wl.timestamps[a:b], delay=delay,
                                    window=window, static_bidirectional=bidir)
            total += int(vis.sum())
            nqt, nkt = -(-L // 128), -(-L // 64)
            cnt = plan["tile_count"][off:off + nqt * nkt].reshape(nqt, nkt)
            for qt in range(nqt):
                ks = plan["ktile_idx"][plan["qtile_ptr"][q]:plan["qtile_ptr"][q + 1]]
                assert np.array_equal(ks, np.nonzero(cnt[qt])[0])
                assert np.all(np.diff(ks) > 0)
                q += 1
            off += nqt * nkt
        assert plan["visible_pairs"] == total
        assert off == plan["tile_count"].shape[0]
        assert np.array_equal(plan["tile_class"] == oracle.EMPTY, plan["tile_count"] == 0)
        assert np.array_equal(plan["tile_class"] == oracle.FULL, plan["tile_count"] == 8192)


def test_serving_plan_total():
    wl = make_config(3, with_qkv=False)
    sub = make_custom([[(HISTORY, wl.timestamps[:2048]), (CANDIDATE, wl.timestamps[2048:2560])]],
                      heads=1, d_head=8, with_qkv=False, window=256)
    plan = oracle.tile_plan(sub.req_offsets, sub.seg_kind, sub.timestamps, delay=0, window=256,
                            static_bidirectional=False)
    assert plan["visible_pairs"] == 1_540_736
    # 20 q-tiles x 40 k-tiles
    assert plan["tile_count"].shape[0] == 800
