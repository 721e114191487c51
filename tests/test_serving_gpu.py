"""Serving call (HSTU, App. H, M-FALCON; CADET "how to score hundreds of
candidates"): history K rotated once into a cache, candidate K rotated per
call, attention computed for the candidates' query tiles only.

* The candidates-only schedule covers exactly the (query tile, head) items
  whose tile holds a CANDIDATE row.
* Those rows are bit-identical to the full call (same tiles, same order)
  unless the item's key range was split (then within a rounding step of it)
  and match the oracle; every other row of O / LSE is left untouched.
* Kind-filtered rotation: rotating PROFILE+HISTORY+REALTIME, then CANDIDATE,
  in place, gives the same bits as rotating everything at once, and rows of
  other kinds are left untouched.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from rk_workloads import (CANDIDATE, HISTORY, PROFILE, REALTIME, make_config,  # noqa: E402
                          make_custom, random_layout)
from test_split_gpu import assert_close_to_unsplit, check_work_list  # noqa: E402

pytestmark = pytest.mark.gpu

BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 1e-2
SENTINEL_I16 = 0x7FC1  # as bf16 bits: a NaN no kernel writes


@pytest.fixture(scope="module")
def rk():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import masked_attention_amd as m
    from masked_attention_amd import _rk
    _rk.lib()
    return m


def _rope(wl):
    return dict(phi_min=wl.phi_min, dt_max=wl.dt_max, base=wl.base)


def _candidate_tiles(wl):
    """Request-local q-tiles holding a candidate row, as global q-tile ids."""
    tiles, qt_off = set(), 0
    offs = wl.req_offsets
    for r in range(offs.shape[0] - 1):
        L = int(offs[r + 1] - offs[r])
        kinds = wl.seg_kind[offs[r]:offs[r + 1]]
        cand = np.nonzero(kinds == CANDIDATE)[0]
        if cand.size:
            for qt in range(int(cand[0]) // 128, (L + 127) // 128):
                tiles.add(qt_off + qt)
        qt_off += (L + 127) // 128
    return tiles


def _rows_of_tiles(wl, tiles):
    rows, qt_off = [], 0
    offs = wl.req_offsets
    for r in range(offs.shape[0] - 1):
        L = int(offs[r + 1] - offs[r])
        for qt in range((L + 127) // 128):
            if qt_off + qt in tiles:
                rows.extend(range(int(offs[r]) + 128 * qt, int(offs[r]) + min(L, 128 * qt + 128)))
        qt_off += (L + 127) // 128
    return np.array(rows, dtype=np.int64)


def _serving_layout(seed):
    rng = np.random.default_rng(seed)
    reqs = random_layout(rng, 5, 700, kinds=(PROFILE, HISTORY, REALTIME, CANDIDATE))
    # make sure most requests have candidates
    reqs += random_layout(rng, 3, 600, kinds=(HISTORY, CANDIDATE), allow_empty=False)
    return reqs


@pytest.mark.parametrize("seed", [0, 1])
def test_candidates_only_schedule(rk, seed):
    wl = make_custom(_serving_layout(400 + seed), heads=3, d_head=64, dtype="bf16", seed=seed)
    batch = rk.Batch.from_workload(wl)
    plan = rk.Plan(batch, num_heads=wl.heads, candidates_only=True)
    sched = plan.sched().cpu().numpy()
    torch.cuda.synchronize()
    items = sched[sched >= 0]
    assert np.unique(items).size == items.size
    got = {(int(i) // wl.heads, int(i) % wl.heads) for i in items}
    want = {(qt, h) for qt in _candidate_tiles(wl) for h in range(wl.heads)}
    assert got == want
    plan.close()


def _outputs(rk, wl, plan, q, k, v, prerotated):
    T, H, d = wl.total_tokens, wl.heads, wl.d_head
    o = torch.full((T, H, d), SENTINEL_I16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    lse = torch.full((H, T), 12345.0, dtype=torch.float32, device="cuda")
    rk.rk_masked_attn_fwd(plan, q, k, v, out=o, lse=lse, rope=_rope(wl), k_prerotated=prerotated)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("which", ["random", "serving-cfg3", "mtgr-cfg4"])
def test_candidates_only_outputs(rk, which):
    if which == "random":
        wl = make_custom(_serving_layout(410), heads=2, d_head=64, dtype="bf16", seed=410,
                         delay=3600)
    elif which == "serving-cfg3":
        wl = make_config(3)
    else:
        wl = make_config(4)
    batch = rk.Batch.from_workload(wl)
    q, k, v = (torch.from_numpy(x).to("cuda").to(torch.bfloat16) for x in (wl.q, wl.k, wl.v))
    kw = dict(delay=wl.delay, window=wl.window, static_bidirectional=wl.static_bidirectional,
              num_heads=wl.heads)
    full_plan = rk.Plan(batch, **kw)
    cand_plan = rk.Plan(batch, candidates_only=True, **kw)

    # the serving flow: history keys rotated once into the cache, candidate
    # keys rotated in place per call
    cache = k.clone()
    rk.rk_time_rope(batch, cache, out=cache, kinds=(PROFILE, HISTORY, REALTIME), **_rope(wl))
    rk.rk_time_rope(batch, cache, out=cache, kinds=(CANDIDATE,), **_rope(wl))
    krot = rk.rk_time_rope(batch, k, **_rope(wl))
    torch.cuda.synchronize()
    assert torch.equal(cache.view(torch.int16), krot.view(torch.int16))

    o_full, l_full = _outputs(rk, wl, full_plan, q, k, v, prerotated=False)
    o_c, l_c = _outputs(rk, wl, cand_plan, q, cache, v, prerotated=True)
    rows = _rows_of_tiles(wl, _candidate_tiles(wl))
    other = np.setdiff1d(np.arange(wl.total_tokens), rows)
    other_t = torch.from_numpy(other).cuda()
    oc16, of16 = o_c.view(torch.int16), o_full.view(torch.int16)
    split = check_work_list(cand_plan, wl.heads)
    for qt in sorted(_candidate_tiles(wl)):
        rt = torch.from_numpy(_rows_of_tiles(wl, {qt})).cuda()
        for h in range(wl.heads):
            if qt * wl.heads + h in split:
                assert_close_to_unsplit(o_c[rt, h], o_full[rt, h], "bf16")
                assert torch.allclose(l_c[h, rt], l_full[h, rt], rtol=0, atol=1e-4)
            else:
                assert torch.equal(oc16[rt, h], of16[rt, h])
                assert torch.equal(l_c[h, rt], l_full[h, rt])
    if other.size:
        assert bool((oc16[other_t] == SENTINEL_I16).all())
        assert bool((l_c[:, other_t] == 12345.0).all())

    # candidate rows against the oracle (sampled for the big workloads)
    kinds = wl.seg_kind
    cand_rows = np.nonzero(kinds == CANDIDATE)[0]
    if cand_rows.size > 300:
        cand_rows = np.random.default_rng(7).choice(cand_rows, 300, replace=False)
    o_np = o_c.float().cpu().numpy().astype(np.float64)
    for h in range(wl.heads):
        ref_o, _ = oracle.attention_rows(wl.req_offsets, wl.seg_kind, wl.timestamps,
                                         wl.q.astype(np.float64), wl.k.astype(np.float64),
                                         wl.v.astype(np.float64), cand_rows, h, delay=wl.delay,
                                         window=wl.window,
                                         static_bidirectional=wl.static_bidirectional,
                                         rope=_rope(wl))
        got = o_np[cand_rows, h]
        err = np.abs(got - ref_o)
        assert err.max() <= BF16_MAX_ABS, err.max()
        assert np.linalg.norm(got - ref_o) <= BF16_REL_L2 * max(np.linalg.norm(ref_o), 1e-30)
    full_plan.close()
    cand_plan.close()


def test_kind_filtered_rotation_leaves_other_rows(rk):
    wl = make_custom(_serving_layout(420), heads=2, d_head=64, dtype="bf16", seed=420)
    batch = rk.Batch.from_workload(wl)
    k = torch.from_numpy(wl.k).to("cuda").to(torch.bfloat16)
    full = rk.rk_time_rope(batch, k, **_rope(wl))
    out = torch.full_like(k, 0).view(torch.int16).fill_(0x1234).view(torch.bfloat16)
    rk.rk_time_rope(batch, k, out=out, kinds=(CANDIDATE, REALTIME), **_rope(wl))
    torch.cuda.synchronize()
    sel = np.isin(wl.seg_kind, (CANDIDATE, REALTIME))
    sel_t = torch.from_numpy(np.nonzero(sel)[0]).cuda()
    oth_t = torch.from_numpy(np.nonzero(~sel)[0]).cuda()
    assert torch.equal(out.view(torch.int16)[sel_t], full.view(torch.int16)[sel_t])
    assert bool((out.view(torch.int16)[oth_t] == 0x1234).all())
