"""GPU parity of HSTU pointwise attention (HSTU eq. 2) through the C ABI
against the CPU fp64 oracle.

Outputs are unnormalised sums over the visible keys, so their magnitude
grows with the row's key count; bounds are relative to it: fp32 within
1e-4 * max(1, max |reference|); bf16 within 2e-2 * max(1, max |reference|)
max-abs and 1e-2 relative L2.  Both bias paths of the MFMA kernel are
covered: short position tables (the bias is constant over most tiles and
enters the product's initial accumulator) and long ones (per-score bias
near the diagonal); time tables whose bucket edges fall inside tiles.
"""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from rk_workloads import (CANDIDATE, HISTORY, NOW, history_span, make_config,  # noqa: E402
                          make_custom, random_layout)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def rk():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import masked_attention_amd as m
    from masked_attention_amd import _rk
    _rk.lib()
    return m


def _check(dtype, got, ref):
    bound_scale = max(1.0, float(np.abs(ref).max()))
    err = np.abs(got - ref).max()
    if dtype == "f32":
        assert err <= 1e-4 * bound_scale, (err, bound_scale)
    else:
        rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
        assert err <= 2e-2 * bound_scale and rel <= 1e-2, (err, bound_scale, rel)


CASES = [("bf16", 64, False, 16, 32), ("bf16", 64, False, 4096, 40), ("bf16", 64, False, 0, 0),
         ("f32", 32, True, 24, 30), ("f32", 64, True, 300, 0), ("f32", 128, True, 0, 20),
         ("bf16", 32, True, 64, 25), ("bf16", 128, True, 8, 12)]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-d{c[1]}-{'ref' if c[2] else 'mfma'}-P{c[3]}-B{c[4]}"
                                             for c in CASES])
def test_pointwise_matches_oracle(rk, case):
    dtype, d, reference, n_pos, n_time = case
    rng = np.random.default_rng(d + n_pos + n_time)
    reqs = random_layout(rng, 4, 700)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    pb = rng.standard_normal(n_pos).astype(np.float32) * 0.5 if n_pos else None
    tb = rng.standard_normal(n_time).astype(np.float32) * 0.5 if n_time else None
    for bidir, delay, window in ((False, 0, 0), (True, 0, 0), (False, 3600, 200)):
        _say(f"[gpu] pointwise {case} bidir={bidir} delay={delay} window={window}")
        wl = make_custom(reqs, heads=2, d_head=d, dtype=dtype, seed=d, delay=delay,
                         window=window, static_bidirectional=bidir)
        batch = rk.Batch.from_workload(wl)
        plan = rk.Plan(batch, delay=delay, window=window, static_bidirectional=bidir,
                       num_heads=2)
        q, k, v = (torch.from_numpy(a).cuda().to(tdt) for a in (wl.q, wl.k, wl.v))
        scale = 1.0 / np.sqrt(d)
        o = rk.rk_pointwise_attn_fwd(
            plan, q, k, v, scale=scale, reference=reference,
            pos_bias=torch.from_numpy(pb).cuda() if pb is not None else None,
            time_bias=torch.from_numpy(tb).cuda() if tb is not None else None)
        torch.cuda.synchronize()
        ref = oracle.pointwise_attention_forward(
            wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q, wl.k, wl.v, delay=delay,
            window=window, static_bidirectional=bidir, scale=float(np.float32(scale)),
            pos_bias=None if pb is None else pb.astype(np.float64),
            time_bias=None if tb is None else tb.astype(np.float64))
        _check(dtype, o.float().cpu().numpy().astype(np.float64), ref)
        plan.close()


def test_pointwise_long_history_fast_and_slow_bias(rk):
    """Long sorted histories: with 32 position buckets almost every tile takes
    the constant-bias path; log2 time buckets change inside some tiles."""
    rng = np.random.default_rng(9)
    reqs = [[(HISTORY, history_span(rng, 3000 - 500 * r, NOW - 60)),
             (CANDIDATE, np.full(7, NOW, np.int64))] for r in range(3)]
    wl = make_custom(reqs, heads=2, d_head=64, dtype="bf16", seed=9)
    pb = (rng.standard_normal(32) * 0.3).astype(np.float32)
    tb = (rng.standard_normal(40) * 0.3).astype(np.float32)
    batch = rk.Batch.from_workload(wl)
    plan = rk.Plan(batch, num_heads=2)
    q, k, v = (torch.from_numpy(a).cuda().to(torch.bfloat16) for a in (wl.q, wl.k, wl.v))
    outs = []
    for reference in (False, True):
        outs.append(rk.rk_pointwise_attn_fwd(plan, q, k, v, scale=0.125, reference=reference,
                                             pos_bias=torch.from_numpy(pb).cuda(),
                                             time_bias=torch.from_numpy(tb).cuda()))
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([rng.choice(wl.total_tokens, 80, replace=False),
                                     np.nonzero(wl.seg_kind == CANDIDATE)[0]]))
    for h in range(2):
        ref = oracle.pointwise_attention_rows(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q,
                                              wl.k, wl.v, toks, h, delay=0, window=0,
                                              static_bidirectional=False, scale=0.125,
                                              pos_bias=pb.astype(np.float64),
                                              time_bias=tb.astype(np.float64))
        for o in outs:
            _check("bf16", o[toks, h].float().cpu().numpy().astype(np.float64), ref)


def test_pointwise_unsorted_history(rk):
    """Histories out of time order are allowed without a delay rule; the
    planner notes them and the MFMA kernel then takes every history tile's
    time range key by key instead of from its end keys.  Time buckets of
    one second: any misjudged range changes a bucket inside a tile."""
    rng = np.random.default_rng(19)
    reqs = []
    for n in (700, 260, 1):
        h = history_span(rng, n, NOW - 60)
        rng.shuffle(h[: n // 2])  # older half shuffled
        reqs.append([(HISTORY, h), (CANDIDATE, np.full(5, NOW, np.int64))])
    wl = make_custom(reqs, heads=2, d_head=64, dtype="bf16", seed=19)
    assert np.any(np.diff(wl.timestamps[:700]) < 0)
    tb = (rng.standard_normal(26) * 0.5).astype(np.float32)
    batch = rk.Batch.from_workload(wl)
    plan = rk.Plan(batch, num_heads=2)
    assert plan.stats()["status"] == 0
    q, k, v = (torch.from_numpy(a).cuda().to(torch.bfloat16) for a in (wl.q, wl.k, wl.v))
    o = rk.rk_pointwise_attn_fwd(plan, q, k, v, scale=0.125, time_bias=torch.from_numpy(tb).cuda())
    torch.cuda.synchronize()
    ref = oracle.pointwise_attention_forward(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q,
                                             wl.k, wl.v, delay=0, window=0,
                                             static_bidirectional=False, scale=0.125,
                                             time_bias=tb.astype(np.float64))
    _check("bf16", o.float().cpu().numpy().astype(np.float64), ref)
    plan.close()


def test_pointwise_workload_sampled(rk):
    """TM20K-shaped batch (8 x (20000 + 1), H = 8), causal, rab tables of 128
    position and 32 time buckets, on sampled rows of two requests."""
    wl = make_config(5)
    rng = np.random.default_rng(5)
    pb = (rng.standard_normal(128) * 0.3).astype(np.float32)
    tb = (rng.standard_normal(32) * 0.3).astype(np.float32)
    batch = rk.Batch.from_workload(wl)
    plan = rk.Plan(batch, num_heads=wl.heads)
    q, k, v = (torch.from_numpy(a).cuda().to(torch.bfloat16) for a in (wl.q, wl.k, wl.v))
    o = rk.rk_pointwise_attn_fwd(plan, q, k, v, scale=0.125, pos_bias=torch.from_numpy(pb).cuda(),
                                 time_bias=torch.from_numpy(tb).cuda())
    torch.cuda.synchronize()
    for r in (0, wl.num_requests - 1):
        a, b = wl.request(r)
        toks = a + np.unique(np.concatenate([[0, 1, b - a - 1], rng.choice(b - a, 40, replace=False)]))
        h = r % wl.heads
        ref = oracle.pointwise_attention_rows(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q,
                                              wl.k, wl.v, toks, h, delay=0, window=0,
                                              static_bidirectional=False, scale=0.125,
                                              pos_bias=pb.astype(np.float64),
                                              time_bias=tb.astype(np.float64))
        _check("bf16", o[toks, h].float().cpu().numpy().astype(np.float64), ref)


def _candidate_tile_rows(wl):
    """Rows of the query tiles (128 rows, request-local) holding a CANDIDATE row."""
    rows = []
    offs = wl.req_offsets
    for r in range(offs.shape[0] - 1):
        a, b = int(offs[r]), int(offs[r + 1])
        cand = np.nonzero(wl.seg_kind[a:b] == CANDIDATE)[0]
        for qt in sorted({int(c) // 128 for c in cand}):
            rows.extend(range(a + 128 * qt, min(b, a + 128 * qt + 128)))
    return np.asarray(rows, dtype=np.int64)


@pytest.mark.parametrize("reference", [False, True], ids=["mfma", "ref"])
def test_pointwise_candidates_only(rk, reference):
    """Serving call (HSTU App. H): a candidates-only plan writes the rows of
    the query tiles holding candidates, bit-identical to the full call (same
    tiles in the same order), and leaves every other row as it was; the
    candidate rows match the oracle."""
    rng = np.random.default_rng(31)
    reqs = [[(HISTORY, history_span(rng, n_hist, NOW - 60)),
             (CANDIDATE, np.full(n_cand, NOW, np.int64))]
            for n_hist, n_cand in ((900, 150), (300, 0), (1500, 40), (64, 64))]
    wl = make_custom(reqs, heads=2, d_head=64, dtype="bf16", seed=31, delay=3600)
    pb = (rng.standard_normal(64) * 0.3).astype(np.float32)
    tb = (rng.standard_normal(32) * 0.3).astype(np.float32)
    bias = dict(pos_bias=torch.from_numpy(pb).cuda(), time_bias=torch.from_numpy(tb).cuda())
    batch = rk.Batch.from_workload(wl)
    full = rk.Plan(batch, delay=wl.delay, num_heads=2)
    cand = rk.Plan(batch, delay=wl.delay, num_heads=2, candidates_only=True)
    q, k, v = (torch.from_numpy(a).cuda().to(torch.bfloat16) for a in (wl.q, wl.k, wl.v))
    sentinel = 0x7FC1  # bf16 bits of a NaN no kernel writes
    outs = []
    for plan in (full, cand):
        o = torch.full(q.shape, sentinel, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        rk.rk_pointwise_attn_fwd(plan, q, k, v, out=o, scale=0.125, reference=reference, **bias)
        outs.append(o)
    torch.cuda.synchronize()
    rows = _candidate_tile_rows(wl)
    other = np.setdiff1d(np.arange(wl.total_tokens), rows)
    o_full, o_c = (o.view(torch.int16) for o in outs)
    rt, ot = torch.from_numpy(rows).cuda(), torch.from_numpy(other).cuda()
    assert torch.equal(o_c[rt], o_full[rt])
    assert bool((o_c[ot] == sentinel).all())
    cand_rows = np.nonzero(wl.seg_kind == CANDIDATE)[0]
    for h in range(2):
        ref = oracle.pointwise_attention_rows(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q,
                                              wl.k, wl.v, cand_rows, h, delay=wl.delay, window=0,
                                              static_bidirectional=False, scale=0.125,
                                              pos_bias=pb.astype(np.float64),
                                              time_bias=tb.astype(np.float64))
        _check("bf16", outs[1][cand_rows, h].float().cpu().numpy().astype(np.float64), ref)
    full.close()
    cand.close()
