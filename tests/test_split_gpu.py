"""Split key ranges of a serving call (candidates-only plans; HSTU, App. H,
M-FALCON; the flash-decoding split of a long key range).

With few (query tile, head) items to run, each item's CSR key range is cut
into chunks run by separate workgroups; a merge pass rescales their partial
softmax results to a common max and sums them.

* With fewer than RK_SPLIT_SLOTS / 2 scheduled items, the work list covers
  every scheduled item's CSR entries exactly once, in schedule order, in
  contiguous chunks whose lengths differ by at most one; split items number
  their partial results consecutively and the split table names them.  With
  more, it mirrors the schedule.
* Outputs of split items match the oracle to the parity bar and the unsplit
  call to a bf16 / fp32 rounding step; unsplit items stay bit-identical.
  Covered for the MFMA kernel (d_head 64 and 128) with Q pre-scaled (time
  RoPE) and raw (no RoPE), and for the plain kernel (fp32 and bf16, d_head
  32, 64 and 128): the three units the kernels keep their running max in.
* Rows that see nothing in any chunk come out as 0 and LSE -inf.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from rk_workloads import (CANDIDATE, DAY, HISTORY, NOW, history_raw, make_config,  # noqa: E402
                          make_custom)

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 1e-2
SENTINEL_I16 = 0x7FC1
SPLIT_SLOTS = 768  # RK_SPLIT_SLOTS


@pytest.fixture(scope="module")
def rk():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import masked_attention_amd as m
    from masked_attention_amd import _rk
    _rk.lib()
    return m


def _long_layout(seed, lens=((2900, 40), (1700, 3), (3300, 130), (600, 9))):
    """Requests of `hist` HISTORY tokens then `cand` candidates: a few
    candidate tiles with long key ranges, the shape splitting is for."""
    rng = np.random.default_rng(seed)
    reqs = []
    for hist, cand in lens:
        h = history_raw(rng, hist, NOW - DAY)
        c = rng.integers(NOW - DAY + 1, NOW + 1, size=cand).astype(np.int64)
        reqs.append([(HISTORY, h), (CANDIDATE, c)])
    return reqs


def _qtile_rows(wl):
    """Global q-tile id -> (first row, end row) as global token indices."""
    out, offs = [], wl.req_offsets
    for r in range(offs.shape[0] - 1):
        a, b = int(offs[r]), int(offs[r + 1])
        for qt in range((b - a + 127) // 128):
            out.append((a + 128 * qt, min(b, a + 128 * qt + 128)))
    return out


def check_work_list(plan, H):
    """Validate the work list against the schedule and CSR; return the
    split items as {item: nparts}."""
    work = plan.work().cpu().numpy()
    splits = plan.splits().cpu().numpy()
    sched = plan.sched().cpu().numpy()
    qptr = plan.qtile_ptr().cpu().numpy()
    st = plan.stats()
    nw, ns = st["work_entries"], st["split_items"]
    assert work.shape[0] == sched.shape[0] + SPLIT_SLOTS
    assert 0 <= nw <= work.shape[0]
    assert (work[nw:, 0] == -1).all()
    items = sched[sched >= 0]
    if items.size >= SPLIT_SLOTS // 2:
        # enough items to fill the chip: whole items, the schedule's own order
        assert nw == sched.shape[0] and ns == 0
        assert (work[:nw, 0] == sched).all()
        assert (work[:nw, 1] == 0).all() and (work[:nw, 2] == -1).all()
        assert (work[:nw, 3] == -1).all()
        assert (splits[:, 0] == -1).all()
        return {}
    pos, split, parts_seen = 0, [], []
    for it in items:
        n = int(qptr[it // H + 1] - qptr[it // H])
        first = pos
        while pos < nw and work[pos, 0] == it:
            pos += 1
        ents = work[first:pos]
        assert ents.shape[0] >= 1, f"item {it} has no work entry"
        assert ents[0, 1] == 0 and ents[-1, 2] == n
        assert (ents[1:, 1] == ents[:-1, 2]).all()
        if ents.shape[0] == 1:
            assert ents[0, 3] == -1
            continue
        lens = ents[:, 2] - ents[:, 1]
        assert lens.min() >= 1 and lens.max() - lens.min() <= 1
        parts = ents[:, 3]
        assert (parts == parts[0] + np.arange(parts.shape[0])).all()
        split.append((int(it), int(parts[0]), int(parts.shape[0])))
        parts_seen.extend(parts.tolist())
    assert pos == nw, "work entries beyond the scheduled items"
    assert ns == len(split)
    assert [tuple(int(x) for x in r[:3]) for r in splits[:ns]] == split
    assert (splits[ns:, 0] == -1).all()
    assert len(set(parts_seen)) == len(parts_seen) and max(parts_seen, default=0) < 2048
    return {it: c for it, _, c in split}


def assert_close_to_unsplit(got, full, dtype):
    """Split vs unsplit output of one item.  With bf16, P is rounded to bf16
    against the chunk's own running max instead of the whole range's: each
    probability moves by up to 2^-9 of itself, which shifts an output by an
    absolute amount (about 1e-4 here) however small it is, and the bf16
    output may then round one step away.  Both calls meet the parity bar
    against the oracle on their own; their difference is held to a tenth of
    that bar (2e-3) plus two bf16 steps.  fp32 outputs differ by rounding
    only."""
    got, full = got.float(), full.float()
    if dtype == "bf16":
        ok = (got - full).abs() <= 2.0 ** -6 * full.abs() + 2e-3
    else:
        ok = (got - full).abs() <= 1e-5 * full.abs() + 1e-6
    assert bool(ok.all()), (got - full).abs().max()


def _run(rk, wl, plan, q, k, v, rope, reference):
    T, H, d = wl.total_tokens, wl.heads, wl.d_head
    if q.dtype == torch.bfloat16:
        o = torch.full((T, H, d), SENTINEL_I16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    else:
        o = torch.full((T, H, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((H, T), 12345.0, dtype=torch.float32, device="cuda")
    rk.rk_masked_attn_fwd(plan, q, k, v, out=o, lse=lse, rope=rope, reference=reference)
    torch.cuda.synchronize()
    return o, lse


CASES = [
    # (dtype, d_head, time RoPE, plain kernel)
    ("bf16", 64, True, False),    # MFMA, Q pre-scaled: max in log2 units
    ("bf16", 64, False, False),   # MFMA, raw scores: max in dot-product units
    ("bf16", 64, True, True),     # plain kernel: max in natural units
    ("f32", 32, True, False),
    ("f32", 128, False, False),
    ("bf16", 128, True, False),   # MFMA at d_head 128 (two-stage form)
    ("bf16", 128, False, False),
    ("bf16", 128, True, True),    # plain kernel at d_head 128
    ("bf16", 88, True, False),    # padded instances: MFMA at 128, plain at 64
    ("f32", 40, True, False),
]


@pytest.mark.parametrize("dtype,d,use_rope,reference", CASES)
def test_split_outputs(rk, dtype, d, use_rope, reference):
    wl = make_custom(_long_layout(500 + d), heads=2, d_head=d, dtype=dtype, seed=500 + d,
                     delay=600, name=f"split-{dtype}-{d}")
    H = wl.heads
    batch = rk.Batch.from_workload(wl)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x).to("cuda").to(tdt) for x in (wl.q, wl.k, wl.v))
    rope = dict(phi_min=wl.phi_min, dt_max=wl.dt_max, base=wl.base) if use_rope else None
    kw = dict(delay=wl.delay, num_heads=H)
    full_plan = rk.Plan(batch, **kw)
    cand_plan = rk.Plan(batch, candidates_only=True, **kw)
    split = check_work_list(cand_plan, H)
    assert split, "layout meant to split produced no split item"

    o_f, l_f = _run(rk, wl, full_plan, q, k, v, rope, reference)
    o_c, l_c = _run(rk, wl, cand_plan, q, k, v, rope, reference)
    tiles = _qtile_rows(wl)
    sched = cand_plan.sched().cpu().numpy()
    bits = (lambda t: t.view(torch.int16)) if dtype == "bf16" else (lambda t: t.view(torch.int32))
    for it in sched[sched >= 0]:
        qt, h = int(it) // H, int(it) % H
        a, b = tiles[qt]
        if it in split:
            assert_close_to_unsplit(o_c[a:b, h], o_f[a:b, h], dtype)
            lf, lc = l_f[h, a:b], l_c[h, a:b]
            assert torch.equal(torch.isinf(lf), torch.isinf(lc))
            fin = torch.isfinite(lf)
            assert torch.allclose(lc[fin], lf[fin], rtol=0, atol=1e-4)
        else:
            assert torch.equal(bits(o_c[a:b, h]), bits(o_f[a:b, h]))
            assert torch.equal(l_c[h, a:b], l_f[h, a:b])

    # every row of a split item against the oracle
    rows_h = {}
    for it in split:
        qt, h = it // H, it % H
        a, b = tiles[qt]
        rows_h.setdefault(h, []).extend(range(a, b))
    oc = o_c.float().cpu().numpy().astype(np.float64)
    lc = l_c.cpu().numpy().astype(np.float64)
    for h, rows in rows_h.items():
        rows = np.array(sorted(rows), np.int64)
        ref_o, ref_l = oracle.attention_rows(
            wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q.astype(np.float64),
            wl.k.astype(np.float64), wl.v.astype(np.float64), rows, h, delay=wl.delay,
            window=0, static_bidirectional=False, rope=rope)
        got = oc[rows, h]
        err = np.abs(got - ref_o)
        if dtype == "bf16":
            assert err.max() <= BF16_MAX_ABS, err.max()
            assert np.linalg.norm(got - ref_o) <= BF16_REL_L2 * max(np.linalg.norm(ref_o), 1e-30)
        else:
            assert err.max() <= F32_TOL, err.max()
        gl = lc[h, rows]
        assert np.array_equal(np.isinf(gl), np.isinf(ref_l))
        fin = np.isfinite(ref_l)
        lse_tol = F32_TOL if dtype == "f32" else BF16_MAX_ABS
        assert np.abs(gl[fin] - ref_l[fin]).max(initial=0.0) <= lse_tol
    full_plan.close()
    cand_plan.close()


def test_split_rows_seeing_nothing(rk):
    """With a delay larger than the whole history span, HISTORY rows inside a
    candidate tile see no key at all (a U2U key needs t_j <= t_i - delay,
    so not even the row itself), in any chunk: they must come out as 0 and
    LSE -inf."""
    rng = np.random.default_rng(520)
    reqs = []
    for hist, cand in ((2000, 20), (2500, 60)):
        # history packed inside one hour: a one-day delay hides all of it
        h = np.sort(rng.integers(NOW - 3600, NOW - 1800, size=hist)).astype(np.int64)
        c = np.full(cand, NOW, np.int64)
        reqs.append([(HISTORY, h), (CANDIDATE, c)])
    wl = make_custom(reqs, heads=2, d_head=64, dtype="bf16", seed=520, delay=DAY,
                     name="split-empty-rows")
    batch = rk.Batch.from_workload(wl)
    q, k, v = (torch.from_numpy(x).to("cuda").to(torch.bfloat16) for x in (wl.q, wl.k, wl.v))
    plan = rk.Plan(batch, delay=wl.delay, num_heads=wl.heads, candidates_only=True)
    split = check_work_list(plan, wl.heads)
    assert split
    rope = dict(phi_min=wl.phi_min, dt_max=wl.dt_max, base=wl.base)
    o, lse = _run(rk, wl, plan, q, k, v, rope, False)
    tiles = _qtile_rows(wl)
    n_empty = 0
    for it in split:
        qt, h = it // wl.heads, it % wl.heads
        a, b = tiles[qt]
        rows = np.arange(a, b)
        ref_o, ref_l = oracle.attention_rows(
            wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q.astype(np.float64),
            wl.k.astype(np.float64), wl.v.astype(np.float64), rows, h, delay=wl.delay,
            window=0, static_bidirectional=False, rope=rope)
        empty = np.isinf(ref_l)
        n_empty += int(empty.sum())
        got_l = lse[h, a:b].cpu().numpy()
        assert np.array_equal(np.isinf(got_l), empty)
        got_o = o[a:b, h].float().cpu().numpy()
        assert (got_o[empty] == 0).all()
        err = np.abs(got_o[~empty] - ref_o[~empty])
        assert err.max(initial=0.0) <= BF16_MAX_ABS
    assert n_empty > 0, "layout meant to hold rows with no visible key has none"
    plan.close()


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 128)])
def test_split_many_parts(rk, dtype, d):
    """One request of 20,000 history keys and one candidate, one head: its
    only item (313 key tiles) splits into ceil(313 / 8) = 40 parts, more than
    the merge reads in one group, so the merge's online rescaling runs over
    several groups and a short last one.  Candidate tile rows against the
    oracle."""
    rng = np.random.default_rng(530)
    h = history_raw(rng, 20000, NOW - DAY)
    reqs = [[(HISTORY, h), (CANDIDATE, np.array([NOW], np.int64))]]
    wl = make_custom(reqs, heads=1, d_head=d, dtype=dtype, seed=530, name="split-40-parts")
    batch = rk.Batch.from_workload(wl)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x).to("cuda").to(tdt) for x in (wl.q, wl.k, wl.v))
    plan = rk.Plan(batch, num_heads=1, candidates_only=True)
    split = check_work_list(plan, 1)
    assert list(split.values()) == [40]
    rope = dict(phi_min=wl.phi_min, dt_max=wl.dt_max, base=wl.base)
    o, lse = _run(rk, wl, plan, q, k, v, rope, False)
    (it,) = split
    a, b = _qtile_rows(wl)[it]
    rows = np.arange(a, b)
    ref_o, ref_l = oracle.attention_rows(
        wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q.astype(np.float64),
        wl.k.astype(np.float64), wl.v.astype(np.float64), rows, 0, delay=0, window=0,
        static_bidirectional=False, rope=rope)
    got_o = o[a:b, 0].float().cpu().numpy()
    got_l = lse[0, a:b].cpu().numpy()
    tol = BF16_MAX_ABS if dtype == "bf16" else F32_TOL
    assert np.abs(got_o - ref_o).max() <= tol * max(1.0, np.abs(ref_o).max())
    assert np.abs(got_l - ref_l).max() <= 1e-3
    plan.close()


@pytest.mark.parametrize("cfg", [3, 5])
def test_split_work_list_workloads(rk, cfg):
    """The serving workload (3: 1024 items, the schedule mirrored) and the
    8 x (20000+1) causal workload (5): work-list invariants on the real
    shapes; on workload 5 every item splits (64 items, 313 key tiles each,
    chunks of at most C = max(8, ceil(total / RK_SPLIT_SLOTS)) tiles)."""
    wl = make_config(cfg, with_qkv=False)
    batch = rk.Batch.from_workload(wl)
    plan = rk.Plan(batch, delay=wl.delay, window=wl.window,
                   static_bidirectional=wl.static_bidirectional, num_heads=wl.heads,
                   candidates_only=True)
    split = check_work_list(plan, wl.heads)
    if cfg == 5:
        C = max(8, -(-64 * 313 // SPLIT_SLOTS))
        c = -(-313 // C)
        assert len(split) == 64 and all(v == c for v in split.values())
        assert plan.stats()["work_entries"] == 64 * c
    else:
        assert not split
    plan.close()
