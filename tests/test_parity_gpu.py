"""GPU parity: the HIP path through the C ABI against the CPU fp64 oracle.

* Plan: tile classes, exact per-tile visible counts, CSR and totals are
  bit-exact; row descriptors reproduce each oracle mask row exactly; the
  launch schedule covers every (query tile, head) once.
* Time RoPE: rotated Q/K against the oracle rotation by (t - anchor).
* Attention: fp32 within 1e-4 max-abs; bf16 within 2e-2 max-abs and 1e-2
  relative L2 against the oracle on the bf16-rounded inputs.  Small batches
  (several tiles, ragged tails, every mask mode) are compared in full; the
  five named workloads at full size, in the launch configuration the
  benchmark times, are compared on sampled rows.
"""

import math
import os
import sys
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from rk_workloads import (CANDIDATE, HISTORY, NOW, PROFILE, REALTIME, make_config,  # noqa: E402
                          make_custom, random_layout)

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 1e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def rk():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import masked_attention_amd as m
    from masked_attention_amd import _rk
    _rk.lib()  # fails loudly if librk.so is missing
    return m


def _rope(wl):
    return dict(phi_min=wl.phi_min, dt_max=wl.dt_max, base=wl.base)


def _tensors(wl):
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    q = torch.from_numpy(wl.q).to("cuda").to(dt)
    k = torch.from_numpy(wl.k).to("cuda").to(dt)
    v = torch.from_numpy(wl.v).to("cuda").to(dt)
    return q, k, v


def _plan(rk, wl, batch=None):
    batch = batch or rk.Batch.from_workload(wl)
    plan = rk.Plan(batch, delay=wl.delay, window=wl.window,
                   static_bidirectional=wl.static_bidirectional, num_heads=wl.heads,
                   global_tail=wl.global_tail)
    return batch, plan


def _run(rk, wl, rope=True, reference=False, want_lse=True):
    _say(f"[gpu] {wl.name}: T={wl.total_tokens} H={wl.heads} d={wl.d_head} {wl.dtype} "
         f"rope={rope} reference={reference}")
    batch, plan = _plan(rk, wl)
    q, k, v = _tensors(wl)
    o, lse = rk.rk_masked_attn_fwd(plan, q, k, v, rope=_rope(wl) if rope else None,
                                   reference=reference, want_lse=want_lse)
    torch.cuda.synchronize()
    o_np = o.float().cpu().numpy().astype(np.float64)
    lse_np = lse.cpu().numpy().astype(np.float64) if lse is not None else None
    return plan, o_np, lse_np


def _oracle_full(wl, rope=True):
    return oracle.attention_forward(wl.req_offsets, wl.seg_kind, wl.timestamps,
                                    wl.q.astype(np.float64), wl.k.astype(np.float64),
                                    wl.v.astype(np.float64), delay=wl.delay, window=wl.window,
                                    static_bidirectional=wl.static_bidirectional,
                                    rope=_rope(wl) if rope else None,
                                    global_tail=wl.global_tail)


def _check(wl, o, ref, lse=None, ref_lse=None):
    err = np.abs(o - ref)
    if wl.dtype == "f32":
        assert err.max() <= F32_TOL, f"max abs {err.max()}"
    else:
        rel = np.linalg.norm(o - ref) / max(np.linalg.norm(ref), 1e-30)
        assert err.max() <= BF16_MAX_ABS, f"max abs {err.max()}"
        assert rel <= BF16_REL_L2, f"rel L2 {rel}"
    if lse is not None:
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.all(np.isneginf(lse[~fin]))
        tol = 1e-4 if wl.dtype == "f32" else 2e-2
        if fin.any():
            assert np.abs(lse[fin] - ref_lse[fin]).max() <= tol


# ---------------------------------------------------------------------------
# plan
# ---------------------------------------------------------------------------

def _check_plan(wl, plan, ref, check_rows=True):
    torch.cuda.synchronize()
    st = plan.stats()
    assert st["device_errors"] == 0
    tc = plan.tile_class().cpu().numpy()
    cnt = plan.tile_count().cpu().numpy()
    assert np.array_equal(tc, ref["tile_class"])
    assert np.array_equal(cnt.astype(np.int64), ref["tile_count"])
    assert np.array_equal(plan.qtile_ptr().cpu().numpy().astype(np.int64), ref["qtile_ptr"])
    assert np.array_equal(plan.ktile_idx().cpu().numpy().astype(np.int64), ref["ktile_idx"])
    assert st["visible_pairs"] == ref["visible_pairs"]
    assert st["full_tiles"] == int((ref["tile_class"] == oracle.FULL).sum())
    assert st["partial_tiles"] == int((ref["tile_class"] == oracle.PARTIAL).sum())
    assert st["empty_tiles"] == int((ref["tile_class"] == oracle.EMPTY).sum())
    # schedule: every (q-tile, head) exactly once, the rest -1
    sched = plan.sched().cpu().numpy()
    items = sched[sched >= 0]
    NQ = plan.num_qtiles
    assert np.array_equal(np.sort(items), np.arange(NQ * wl.heads))
    if check_rows:
        rd = plan.row_desc().cpu().numpy()
        for r in range(wl.num_requests):
            a, b = wl.request(r)
            if b == a:
                continue
            vis = oracle.visibility(wl.seg_kind[a:b], wl.timestamps[a:b], delay=wl.delay,
                                    window=wl.window, static_bidirectional=wl.static_bidirectional,
                                    global_tail=wl.global_tail)
            lo = rd[a:b, 0]
            hi = rd[a:b, 1] & 0x7FFFFFFF
            self_ = rd[a:b, 1] < 0
            cols = np.arange(b - a)[None, :]
            rows = np.arange(b - a)[:, None]
            mine = ((cols >= lo[:, None]) & (cols < hi[:, None])) | (self_[:, None] & (cols == rows))
            assert np.array_equal(mine, vis), f"request {r}"


LAYOUT_CASES = [
    # (name, requests builder, delay, window, bidir)
    ("causal-ragged", lambda rng: [[(HISTORY, np.sort(rng.integers(NOW - 10**7, NOW, 300)))],
                                   [(HISTORY, np.sort(rng.integers(NOW - 10**7, NOW, 129)))],
                                   [(HISTORY, np.sort(rng.integers(NOW - 10**7, NOW, 1)))]], 0, 0, False),
    ("delay-ties", lambda rng: [[(HISTORY, np.sort(rng.integers(NOW - 20000, NOW, 400)))]], 3600, 0, False),
    ("window-cands", lambda rng: [[(HISTORY, np.sort(rng.integers(NOW - 10**7, NOW - 60, 333))),
                                   (CANDIDATE, np.full(70, NOW))]], 0, 37, False),
    ("window-delay", lambda rng: [[(HISTORY, np.sort(rng.integers(NOW - 10**6, NOW - 60, 260))),
                                   (CANDIDATE, np.full(5, NOW))]], 1800, 100, False),
    ("mtgr-small", lambda rng: [[(PROFILE, np.full(5, NOW)),
                                 (HISTORY, np.sort(rng.integers(NOW - 10**7, NOW - 86400, 140))),
                                 (REALTIME, np.sort(rng.integers(NOW - 86400, NOW, 30))),
                                 (CANDIDATE, rng.integers(NOW - 86400, NOW, 21))]], 0, 0, True),
    # profile tokens dated at the anchor ("now") under a causal static part
    # with a delay: the delay rule hides them from the history rows, which
    # then see a history prefix that starts after the profile
    ("profile-at-anchor-delay", lambda rng: [
        [(PROFILE, np.full(40, NOW)),
         (HISTORY, np.sort(rng.integers(NOW - 10**6, NOW - 60, 300))),
         (CANDIDATE, np.full(9, NOW))],
        [(PROFILE, np.full(130, NOW)), (HISTORY, np.sort(rng.integers(NOW - 10**5, NOW, 200)))],
        [(PROFILE, np.full(7, NOW))]], 3600, 0, False),
    ("profile-at-anchor-window-delay", lambda rng: [
        [(PROFILE, np.full(70, NOW)),
         (HISTORY, np.sort(rng.integers(NOW - 10**6, NOW - 60, 400))),
         (REALTIME, np.sort(rng.integers(NOW - 50, NOW, 12))),
         (CANDIDATE, rng.integers(NOW - 50, NOW, 20))]], 600, 100, False),
    ("empty-and-tiny", lambda rng: [[], [(CANDIDATE, np.full(3, NOW))], [],
                                    [(HISTORY, np.array([NOW - 5])), (CANDIDATE, np.array([NOW]))],
                                    [(HISTORY, np.sort(rng.integers(NOW - 10**5, NOW, 128)))]], 0, 0, False),
]


@pytest.mark.parametrize("case", LAYOUT_CASES, ids=[c[0] for c in LAYOUT_CASES])
def test_plan_bit_exact_small(rk, case):
    name, build, delay, window, bidir = case
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    wl = make_custom(build(rng), heads=3, d_head=64, dtype="bf16", delay=delay, window=window,
                     static_bidirectional=bidir, with_qkv=False, name=name)
    _say(f"[gpu] plan {name}")
    batch, plan = _plan(rk, wl)
    ref = oracle.tile_plan(wl.req_offsets, wl.seg_kind, wl.timestamps, delay=delay,
                           window=window, static_bidirectional=bidir)
    _check_plan(wl, plan, ref)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_plan_bit_exact_random(rk, seed):
    rng = np.random.default_rng(100 + seed)
    reqs = random_layout(rng, 7, 700)
    for bidir, delay, window in ((True, 0, 0), (False, 3600, 0), (False, 0, 50), (False, 7200, 200)):
        wl = make_custom(reqs, heads=2, d_head=64, dtype="bf16", delay=delay, window=window,
                         static_bidirectional=bidir, with_qkv=False)
        _say(f"[gpu] plan random seed={seed} bidir={bidir} delay={delay} window={window}")
        batch, plan = _plan(rk, wl)
        ref = oracle.tile_plan(wl.req_offsets, wl.seg_kind, wl.timestamps, delay=delay,
                               window=window, static_bidirectional=bidir)
        _check_plan(wl, plan, ref)


def test_plans_queued_ahead_of_the_gpu(rk):
    """Plans issued while the stream is still busy: each one's host tables
    wait in a pinned host block until its first planner kernel reads them,
    so 80 plans in flight take every block the library keeps (then fall back
    to an asynchronous copy); blocks are reused once read.  Every plan,
    whichever way its tables went up, is bit-exact, and so is a second round
    that reuses the blocks."""
    rng = np.random.default_rng(11)
    reqs = random_layout(rng, 5, 600)
    wl = make_custom(reqs, heads=2, d_head=64, dtype="bf16", delay=3600, with_qkv=False,
                     name="queued")
    ref = oracle.tile_plan(wl.req_offsets, wl.seg_kind, wl.timestamps, delay=wl.delay, window=0,
                           static_bidirectional=False)
    batch = rk.Batch.from_workload(wl)
    for rnd in range(2):
        _say(f"[gpu] plans queued ahead, round {rnd}")
        torch.cuda.synchronize()
        torch.cuda._sleep(100_000_000)  # the stream stays busy while the plans are issued
        plans = [rk.Plan(batch, delay=wl.delay, num_heads=wl.heads) for _ in range(80)]
        for i, plan in enumerate(plans):
            _check_plan(wl, plan, ref, check_rows=(i % 16 == 0 or i == len(plans) - 1))
            plan.close()


def test_plans_from_several_host_threads(rk):
    """Plans built from four host threads at once, each on its own stream:
    the pinned host blocks are handed out under a lock, so every plan gets
    its own tables and all of them are bit-exact."""
    import threading
    rng = np.random.default_rng(13)
    reqs = random_layout(rng, 6, 700)
    wl = make_custom(reqs, heads=2, d_head=64, dtype="bf16", delay=1800, window=300,
                     with_qkv=False, name="threads")
    ref = oracle.tile_plan(wl.req_offsets, wl.seg_kind, wl.timestamps, delay=wl.delay,
                           window=wl.window, static_bidirectional=False)
    batch = rk.Batch.from_workload(wl)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(4)]
    plans = [[] for _ in streams]
    errors = []

    def work(i):
        try:
            for _ in range(12):
                plans[i].append(rk.Plan(batch, delay=wl.delay, window=wl.window,
                                        num_heads=wl.heads, stream=streams[i]))
        except Exception as e:  # reported below, in the test's own thread
            errors.append(e)

    _say("[gpu] plans from four host threads")
    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(streams))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for i, ps in enumerate(plans):
        assert len(ps) == 12
        for j, plan in enumerate(ps):
            _check_plan(wl, plan, ref, check_rows=(j == 0))
            plan.close()


def test_plan_captured_in_graph(rk):
    """A plan built under stream capture: its host tables then go up by a
    copy from the plan's own buffer (a pinned block could hold another
    plan's tables by the time a replay runs).  Three replays, with eager
    plans built and the workspace cleared between them, are each
    bit-exact."""
    rng = np.random.default_rng(12)
    reqs = random_layout(rng, 4, 500)
    wl = make_custom(reqs, heads=2, d_head=64, dtype="bf16", delay=3600, with_qkv=False,
                     name="graph")
    ref = oracle.tile_plan(wl.req_offsets, wl.seg_kind, wl.timestamps, delay=wl.delay, window=0,
                           static_bidirectional=False)
    batch = rk.Batch.from_workload(wl)
    size = rk.binding.rk_plan_workspace_size(batch, wl.heads)
    ws = torch.zeros(max(size, 256), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=side):
        plan = rk.Plan(batch, delay=wl.delay, num_heads=wl.heads, workspace=ws)
    torch.cuda.synchronize()
    for rnd in range(3):
        _say(f"[gpu] captured plan, replay {rnd}")
        ws.zero_()
        others = [rk.Plan(batch, delay=wl.delay, num_heads=wl.heads) for _ in range(3)]
        graph.replay()
        torch.cuda.synchronize()
        _check_plan(wl, plan, ref, check_rows=(rnd == 0))
        for o in others:
            _check_plan(wl, o, ref, check_rows=False)
            o.close()
    plan.close()
    del graph


@pytest.mark.parametrize("delay,window,bidir", [(0, 0, False), (3600, 0, False), (0, 300, False),
                                                 (1800, 1000, False), (0, 0, True)])
def test_plan_bit_exact_lengths(rk, delay, window, bidir):
    """Requests whose k-tile counts give every split of a tile's rows over
    lanes in the tile-count kernel (1 to 64 lanes per k-tile: 129+, 65-128,
    33-64, 17-32, 9-16, 5-8, 3-4 and 1-2 k-tiles), with candidates and
    real-time tokens, counted bit-exactly against the oracle."""
    rng = np.random.default_rng(7 + delay + window + bidir)
    reqs = []
    for n in (9000, 5000, 3000, 1500, 700, 400, 200, 100, 1):
        hist = np.sort(rng.integers(NOW - 10**6, NOW - 3600, n)).astype(np.int64)
        rt = np.sort(rng.integers(NOW - 3600, NOW, 40)).astype(np.int64)
        reqs.append([(HISTORY, hist), (REALTIME, rt), (CANDIDATE, np.full(25, NOW, np.int64))])
    wl = make_custom(reqs, heads=2, d_head=64, dtype="bf16", delay=delay, window=window,
                     static_bidirectional=bidir, with_qkv=False, name="lengths")
    _say(f"[gpu] plan lengths delay={delay} window={window} bidir={bidir}")
    batch, plan = _plan(rk, wl)
    ref = oracle.tile_plan(wl.req_offsets, wl.seg_kind, wl.timestamps, delay=delay,
                           window=window, static_bidirectional=bidir)
    _check_plan(wl, plan, ref)
    plan.close()


@pytest.mark.parametrize("G", [1, 37, 300])
def test_plan_and_attention_global_tail(rk, G):
    """LazFormer global-tail queries (eq. 19-21, G > 0) with a window and a
    delay: plan bit-exact (row descriptors included), attention within the
    bf16 bar."""
    rng = np.random.default_rng(500 + G)
    reqs = random_layout(rng, 6, 900)
    for window, delay in ((40, 0), (100, 3600)):
        wl = make_custom(reqs, heads=2, d_head=64, dtype="bf16", delay=delay, window=window,
                         global_tail=G, seed=G, name=f"global-tail-{G}-{window}")
        _say(f"[gpu] global tail G={G} window={window} delay={delay}")
        batch, plan = _plan(rk, wl)
        ref = oracle.tile_plan(wl.req_offsets, wl.seg_kind, wl.timestamps, delay=delay,
                               window=window, static_bidirectional=False, global_tail=G)
        _check_plan(wl, plan, ref)
        plan2, o, lse = _run(rk, wl)
        ref_o, ref_lse = _oracle_full(wl)
        _check(wl, o, ref_o, lse, ref_lse)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_plan_bit_exact_workloads(rk, cfg):
    wl = make_config(cfg, with_qkv=False)
    _say(f"[gpu] plan workload {cfg}")
    batch, plan = _plan(rk, wl)
    ref = oracle.tile_plan(wl.req_offsets, wl.seg_kind, wl.timestamps, delay=wl.delay,
                           window=wl.window, static_bidirectional=wl.static_bidirectional)
    _check_plan(wl, plan, ref, check_rows=cfg in (1, 2))


def test_plan_bit_exact_tm20k(rk):
    """Delta = 0: the mask depends on positions only, so every request of the
    long-sequence workload has request 0's tiles."""
    wl = make_config(5, with_qkv=False)
    _say("[gpu] plan workload 5")
    batch, plan = _plan(rk, wl)
    a, b = wl.request(0)
    cnt, cls = oracle.tile_plan_request(wl.seg_kind[a:b], wl.timestamps[a:b], delay=0, window=0,
                                        static_bidirectional=False)
    torch.cuda.synchronize()
    st = plan.stats()
    assert st["visible_pairs"] == 8 * 200_030_001
    n = cnt.size
    gc = plan.tile_count().cpu().numpy().reshape(8, n)
    gk = plan.tile_class().cpu().numpy().reshape(8, n)
    for r in range(8):
        assert np.array_equal(gc[r].astype(np.int64), cnt.ravel())
        assert np.array_equal(gk[r], cls.ravel())
    ptr = plan.qtile_ptr().cpu().numpy()
    idx = plan.ktile_idx().cpu().numpy()
    for g in range(0, plan.num_qtiles, 13):
        qt = g % cnt.shape[0]
        assert np.array_equal(idx[ptr[g]:ptr[g + 1]], np.nonzero(cnt[qt])[0])


def test_plan_device_checks(rk):
    """Out-of-order segments and unsorted real-time times are reported."""
    ts = np.array([NOW - 10, NOW - 5, NOW - 7, NOW], np.int64)
    bad_kind = make_custom([[(HISTORY, ts[:2]), (REALTIME, ts[2:3]), (HISTORY, ts[3:])]], heads=1,
                           d_head=64, with_qkv=False)
    batch, plan = _plan(rk, bad_kind)
    assert plan.stats(raise_on_error=False)["status"] == 2
    bad_time = make_custom([[(REALTIME, np.array([NOW - 1, NOW - 3])),
                             (CANDIDATE, np.array([NOW]))]], heads=1, d_head=64, with_qkv=False)
    batch, plan = _plan(rk, bad_time)
    assert plan.stats(raise_on_error=False)["status"] == 3
    ok = make_custom([[(HISTORY, np.array([NOW - 1, NOW - 3]))]], heads=1, d_head=64,
                     with_qkv=False)  # unsorted history with delay 0 is allowed
    batch, plan = _plan(rk, ok)
    assert plan.stats()["status"] == 0


def test_plan_static_time_checks(rk):
    """Causal static part with a delay: PROFILE and HISTORY must each be in
    time order (not across the two: profile tokens dated at the anchor are
    accepted), and a row whose delayed keys would form two runs (profile
    times interleaved with history times) is rejected."""
    def status(reqs, delay, bidir=False):
        wl = make_custom(reqs, heads=1, d_head=64, delay=delay, static_bidirectional=bidir,
                         with_qkv=False)
        batch, plan = _plan(rk, wl)
        st = plan.stats(raise_on_error=False)
        plan.close()
        return st["status"], st["device_errors"]

    day = 86400
    hist = np.array([NOW - 50 * day, NOW - 40 * day, NOW - 30 * day, NOW - 20 * day])
    # profile at the anchor, history before it: one run per row, accepted
    assert status([[(PROFILE, np.full(3, NOW)), (HISTORY, hist)]], 3600) == (0, 0)
    # out of order inside HISTORY, or inside PROFILE, with a delay
    assert status([[(HISTORY, hist[::-1])]], 3600) == (3, 2)
    assert status([[(PROFILE, np.array([NOW, NOW - day])), (HISTORY, hist)]], 3600) == (3, 2)
    # the same layouts without a delay, or with a bidirectional static part
    assert status([[(HISTORY, hist[::-1])]], 0)[0] == 0
    assert status([[(PROFILE, np.array([NOW, NOW - day])), (HISTORY, hist)]], 3600, True)[0] == 0
    # profile dated [60 d ago, now]: the history row at 30 d sees the first
    # profile token and the history before it, two runs
    prof = np.array([NOW - 60 * day, NOW])
    assert status([[(PROFILE, prof), (HISTORY, hist)]], 3600) == (3, 4)
    # dated [45 d ago, now]: the rows at 40 d and 30 d see profile token 0
    # and the older history, two runs again
    assert status([[(PROFILE, np.array([NOW - 45 * day, NOW])), (HISTORY, hist)]], 3600)[0] == 3
    # dated [60 d ago, now] with a window of 2: the 30 d row's window holds
    # history only, one run
    wl = make_custom([[(PROFILE, prof), (HISTORY, hist)]], heads=1, d_head=64, delay=3600,
                     window=2, with_qkv=False)
    batch, plan = _plan(rk, wl)
    ref = oracle.tile_plan(wl.req_offsets, wl.seg_kind, wl.timestamps, delay=3600, window=2,
                           static_bidirectional=False)
    _check_plan(wl, plan, ref)
    plan.close()


def test_failed_plan_outputs_nan(rk):
    """A plan whose device checks failed (real-time events out of time order)
    makes every kernel over it store NaN: forward O and LSE (MFMA and plain
    kernels, and the merge of split key ranges), the backward's dQ, dK, dV
    and the pointwise form."""
    from rk_workloads import draw_grad
    rng = np.random.default_rng(29)
    # 3000 history keys: the candidate tile's key range is long enough to split
    reqs = [[(HISTORY, np.sort(rng.integers(NOW - 10**6, NOW - 3600, 3000))),
             (REALTIME, np.array([NOW - 100, NOW - 500, NOW - 200])),
             (CANDIDATE, np.full(5, NOW))],
            [(HISTORY, np.sort(rng.integers(NOW - 10**6, NOW, 200)))]]
    for dtype, reference in (("bf16", False), ("f32", True)):
        _say(f"[gpu] failed plan {dtype} reference={reference}")
        wl = make_custom(reqs, heads=2, d_head=64, dtype=dtype, seed=29)
        batch = rk.Batch.from_workload(wl)
        plan = rk.Plan(batch, num_heads=2, backward=True)
        assert plan.stats(raise_on_error=False)["status"] == 3
        q, k, v = _tensors(wl)
        do = torch.from_numpy(draw_grad(wl)).to("cuda").to(q.dtype)
        o, lse = rk.rk_masked_attn_fwd(plan, q, k, v, rope=_rope(wl), reference=reference,
                                       want_lse=True)
        dq, dk, dv = rk.rk_masked_attn_bwd(plan, q, k, v, o, lse, do, rope=_rope(wl),
                                           reference=reference)
        po = rk.rk_pointwise_attn_fwd(plan, q, k, v, scale=0.125, reference=reference)
        torch.cuda.synchronize()
        for name, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv),
                        ("pointwise", po)):
            assert bool(torch.isnan(t.float()).all()), name
        plan.close()
        # a serving call whose few candidate tiles are split and merged
        cplan = rk.Plan(batch, num_heads=2, candidates_only=True)
        assert cplan.stats(raise_on_error=False)["split_items"] > 0
        o2 = torch.zeros_like(q)
        rk.rk_masked_attn_fwd(cplan, q, k, v, out=o2, rope=_rope(wl), reference=reference)
        torch.cuda.synchronize()
        cand = torch.from_numpy(np.nonzero(wl.seg_kind == CANDIDATE)[0]).cuda()
        assert bool(torch.isnan(o2[cand].float()).all())
        cplan.close()


# ---------------------------------------------------------------------------
# time RoPE
# ---------------------------------------------------------------------------

# heads 3, 6 and 9: the vector pass loads heads in chunks of four (a partial chunk, one full
# and one partial, two full and one partial)
@pytest.mark.parametrize("dtype,d,heads", [("f32", 32, 2), ("bf16", 64, 3), ("f32", 128, 3),
                                           ("bf16", 64, 6), ("f32", 64, 9)])
def test_time_rope_matches_oracle(rk, dtype, d, heads):
    wl = make_config(1) if dtype == "f32" and d == 32 else make_custom(
        random_layout(np.random.default_rng(5), 4, 300), heads=heads, d_head=d, dtype=dtype,
        seed=4)
    _say(f"[gpu] rope {dtype} d={d} heads={heads}")
    batch = rk.Batch.from_workload(wl)
    q, k, v = _tensors(wl)
    out = rk.rk_time_rope(batch, k, **_rope(wl))
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    rel_t = (wl.timestamps - np.repeat(wl.anchors, np.diff(wl.req_offsets))).astype(np.float64)
    ref = oracle.time_rope(wl.k.astype(np.float64), rel_t, **_rope(wl))
    if dtype == "f32":
        assert np.abs(got - ref).max() <= 2e-6
    else:
        # one bf16 rounding of the rotated value
        assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0**-8 + 1e-6)
    # in place gives the same result
    k2 = k.clone()
    rk.rk_time_rope(batch, k2, out=k2, **_rope(wl))
    torch.cuda.synchronize()
    assert torch.equal(k2, out)


# ---------------------------------------------------------------------------
# attention: small batches compared in full
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", LAYOUT_CASES, ids=[c[0] for c in LAYOUT_CASES])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attention_small_full(rk, case, dtype):
    name, build, delay, window, bidir = case
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    wl = make_custom(build(rng), heads=2, d_head=64, dtype=dtype, delay=delay, window=window,
                     static_bidirectional=bidir, seed=17, name=name)
    plan, o, lse = _run(rk, wl)
    ref, ref_lse = _oracle_full(wl)
    _check(wl, o, ref, lse, ref_lse)


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_attention_random_layouts(rk, seed, d):
    rng = np.random.default_rng(200 + seed)
    reqs = random_layout(rng, 5, 520)
    for dtype in ("bf16", "f32"):
        for bidir, delay, window in ((True, 0, 0), (False, 3600, 0), (False, 0, 90)):
            wl = make_custom(reqs, heads=2, d_head=d, dtype=dtype, delay=delay, window=window,
                             static_bidirectional=bidir, seed=seed)
            plan, o, lse = _run(rk, wl)
            ref, ref_lse = _oracle_full(wl)
            _check(wl, o, ref, lse, ref_lse)


@pytest.mark.parametrize("d", [64, 128])
def test_attention_without_rope(rk, d):
    wl = make_custom(random_layout(np.random.default_rng(9), 3, 400), heads=2, d_head=d,
                     dtype="bf16", seed=9, delay=600)
    plan, o, lse = _run(rk, wl, rope=False)
    ref, ref_lse = _oracle_full(wl, rope=False)
    _check(wl, o, ref, lse, ref_lse)


@pytest.mark.parametrize("d", [64, 128])
def test_mfma_and_reference_kernels_agree(rk, d):
    wl = make_custom(random_layout(np.random.default_rng(10), 4, 600), heads=2, d_head=d,
                     dtype="bf16", seed=10, window=77)
    _, o1, l1 = _run(rk, wl)
    _, o2, l2 = _run(rk, wl, reference=True)
    ref, ref_lse = _oracle_full(wl)
    _check(wl, o1, ref, l1, ref_lse)
    _check(wl, o2, ref, l2, ref_lse)


def test_deterministic(rk):
    wl = make_config(2)
    _, o1, _ = _run(rk, wl, want_lse=False)
    _, o2, _ = _run(rk, wl, want_lse=False)
    assert np.array_equal(o1, o2)


def test_strided_inputs(rk):
    """Q, K, V as views of one packed [T, 3, H, d] buffer."""
    wl = make_custom(random_layout(np.random.default_rng(11), 3, 300), heads=2, d_head=64,
                     dtype="bf16", seed=11, delay=3600)
    batch, plan = _plan(rk, wl)
    qkv = torch.from_numpy(np.stack([wl.q, wl.k, wl.v], axis=1)).to("cuda").to(torch.bfloat16)
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    o, lse = rk.rk_masked_attn_fwd(plan, q, k, v, rope=_rope(wl), want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = _oracle_full(wl)
    _check(wl, o.float().cpu().numpy().astype(np.float64), ref,
           lse.cpu().numpy().astype(np.float64), ref_lse)


# ---------------------------------------------------------------------------
# attention: the five workloads at full size, in the benchmark's launch
# configuration (plan, K rotated by a pass, Q rotated while staged)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_attention_workloads_full(rk, cfg):
    """The four smaller workloads compared element by element (every row,
    head and dimension, and every LSE) against the oracle, a few requests
    per oracle call."""
    wl = make_config(cfg)
    plan, o, lse = _run(rk, wl)
    R, offs = wl.num_requests, wl.req_offsets
    step = max(1, R // 8)
    for r0 in range(0, R, step):
        r1 = min(R, r0 + step)
        ref, ref_lse = oracle.attention_forward(
            wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q, wl.k, wl.v, delay=wl.delay,
            window=wl.window, static_bidirectional=wl.static_bidirectional, rope=_rope(wl),
            requests=np.arange(r0, r1))
        a, b = int(offs[r0]), int(offs[r1])
        _check(wl, o[a:b], ref[a:b], lse[:, a:b], ref_lse[:, a:b])
        _say(f"[gpu] workload {cfg}: requests {r0}..{r1 - 1} match")
    # fully masked rows (delay rule) are exactly zero
    if wl.delay > 0:
        for r in range(R):
            a = wl.request(r)[0]
            assert np.all(o[a] == 0.0) and np.all(np.isneginf(lse[:, a]))


def _item_edge_tokens(wl):
    """Per (request, query tile): its first and last valid rows and the
    first row of each of the tile's four waves' boundaries (rows 0, 63, 64,
    127 of the tile, clipped to the request), so that every (request, head,
    query tile) work item and every wave of it is compared."""
    toks = []
    for r in range(wl.num_requests):
        a, b = wl.request(r)
        L = b - a
        for t0 in range(0, L, 128):
            for off in (0, 63, 64, 127):
                toks.append(a + min(t0 + off, L - 1))
    return np.unique(np.array(toks, np.int64))


def test_attention_tm20k_every_item(rk):
    """The TM20K-shaped workload (8 x (20000 + 1), H = 8): rows 0, 63, 64
    and 127 of every query tile (the last valid row for the ragged last
    tile) of every request and head, about 5,000 rows per head."""
    wl = make_config(5)
    plan, o, lse = _run(rk, wl)
    toks = _item_edge_tokens(wl)
    assert toks.shape[0] > 4000
    for h in range(wl.heads):
        ref, ref_lse = oracle.attention_rows(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q,
                                             wl.k, wl.v, toks, h, delay=wl.delay,
                                             window=wl.window,
                                             static_bidirectional=wl.static_bidirectional,
                                             rope=_rope(wl))
        _check(wl, o[toks, h], ref, lse[h, toks], ref_lse)
        _say(f"[gpu] workload 5 head {h}: {toks.shape[0]} rows match")


@pytest.mark.parametrize("d", [8, 40, 88, 120])
def test_attention_padded_d_head(rk, d):
    """d_head that is not an instance width (CADET's 88 among them) runs at
    the next width with zero columns: bf16 on the matrix cores (64 or 128)
    and on the plain kernel, fp32 on the plain kernel, each against the
    oracle.  O is a strided view whose head rows are followed by 8 sentinel
    columns that must stay untouched."""
    rng = np.random.default_rng(880 + d)
    reqs = random_layout(rng, 4, 500)
    for dtype, reference in (("bf16", False), ("bf16", True), ("f32", False)):
        wl = make_custom(reqs, heads=2, d_head=d, dtype=dtype, delay=3600, seed=d,
                         name=f"padded-d{d}")
        _say(f"[gpu] padded d={d} {dtype} reference={reference}")
        batch, plan = _plan(rk, wl)
        q, k, v = _tensors(wl)
        T, H = wl.total_tokens, wl.heads
        big = torch.full((T, H, d + 8), float("nan"), dtype=q.dtype, device="cuda")
        o, lse = rk.rk_masked_attn_fwd(plan, q, k, v, out=big[:, :, :d], rope=_rope(wl),
                                       reference=reference, want_lse=True)
        torch.cuda.synchronize()
        assert bool(torch.isnan(big[:, :, d:].float()).all()), "padding columns written"
        ref, ref_lse = _oracle_full(wl)
        _check(wl, o.float().cpu().numpy().astype(np.float64), ref,
               lse.cpu().numpy().astype(np.float64), ref_lse)
        plan.close()


def test_attention_d128_every_item(rk):
    """bf16 with d_head = 128 (the MFMA kernel's two-stage form): four heads
    over requests of 1,500 to 6,000 history tokens with realtime events and
    candidates under a one-hour delay; rows 0, 63, 64 and 127 of every query
    tile of every request and head against the oracle."""
    rng = np.random.default_rng(128)
    reqs = []
    for lh, nr, nc in ((6000, 40, 64), (1500, 0, 200), (3900, 120, 1), (4500, 7, 33)):
        hist = np.sort(rng.integers(NOW - 10**7, NOW - 60, lh)).astype(np.int64)
        segs = [(HISTORY, hist)]
        if nr:
            segs.append((REALTIME, np.sort(rng.integers(NOW - 7200, NOW, nr)).astype(np.int64)))
        segs.append((CANDIDATE, np.full(nc, NOW, np.int64)))
        reqs.append(segs)
    wl = make_custom(reqs, heads=4, d_head=128, dtype="bf16", seed=128, delay=3600,
                     name="d128-every-item")
    plan, o, lse = _run(rk, wl)
    toks = _item_edge_tokens(wl)
    for h in range(wl.heads):
        ref, ref_lse = oracle.attention_rows(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q,
                                             wl.k, wl.v, toks, h, delay=wl.delay,
                                             window=wl.window,
                                             static_bidirectional=wl.static_bidirectional,
                                             rope=_rope(wl))
        _check(wl, o[toks, h], ref, lse[h, toks], ref_lse)
        _say(f"[gpu] d128 head {h}: {toks.shape[0]} rows match")


@pytest.mark.parametrize("delay,window", [(0, 0), (3600, 4096)])
def test_attention_long_request(rk, delay, window):
    """One request of 131,072 history tokens and 64 candidates (2048 k-tiles
    per q-tile row, 8.6e9 visible pairs per head: past 32-bit counts).  The
    plan's total is checked against the closed form when no delay or
    window applies (causal history L (L + 1) / 2, each candidate L keys and
    itself); sampled output rows against the oracle."""
    rng = np.random.default_rng(131 + delay)
    Lh, Nc = 131072, 64
    hist = np.sort(rng.integers(NOW - 10**8, NOW - 60, Lh)).astype(np.int64)
    wl = make_custom([[(HISTORY, hist), (CANDIDATE, np.full(Nc, NOW, np.int64))]], heads=2,
                     d_head=64, dtype="bf16", seed=131, delay=delay, window=window,
                     name="long-request")
    plan, o, lse = _run(rk, wl)
    st = plan.stats()
    assert st["device_errors"] == 0
    if delay == 0 and window == 0:
        assert st["visible_pairs"] == Lh * (Lh + 1) // 2 + Nc * (Lh + 1)
    toks = np.unique(np.concatenate([
        np.array([0, 1, 63, 64, 127, 128, 4095, 4096, 65535, 65536, Lh - 1, Lh, Lh + Nc - 1]),
        rng.integers(0, Lh + Nc, 24)])).astype(np.int64)
    for h in range(wl.heads):
        ref, ref_lse = oracle.attention_rows(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q,
                                             wl.k, wl.v, toks, h, delay=delay, window=window,
                                             static_bidirectional=False, rope=_rope(wl))
        _check(wl, o[toks, h], ref, lse[h, toks], ref_lse)
    plan.close()


def test_prerotated_k_matches_fused_path(rk):
    """rk_time_rope on K followed by the attention with RK_ATTN_K_PREROTATED
    gives the same bits as the attention rotating K itself."""
    wl = make_custom(random_layout(np.random.default_rng(12), 3, 500), heads=2, d_head=64,
                     dtype="bf16", seed=12, delay=3600)
    batch, plan = _plan(rk, wl)
    q, k, v = _tensors(wl)
    o1, _ = rk.rk_masked_attn_fwd(plan, q, k, v, rope=_rope(wl))
    krot = rk.rk_time_rope(batch, k, **_rope(wl))
    o2, _ = rk.rk_masked_attn_fwd(plan, q, krot, v, rope=_rope(wl), k_prerotated=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("rope", [True, False], ids=["rope", "norope"])
def test_attention_dominant_key(rk, rope):
    """One key per request whose score exceeds every earlier score of the
    rows that see it by far more than 32 log2 units, placed several tiles
    into the request: the running max then jumps mid-row, and every row
    that sees the key must come out as that key's value row.  The query
    offset and the key sit in dimensions 0..7, the four lowest-frequency
    time RoPE pairs, which turn by < 1e-3 rad over the request's time span."""
    rng = np.random.default_rng(31)
    reqs = [
        [(HISTORY, np.sort(rng.integers(NOW - 300 * 86400, NOW - 86400, 700))),
         (REALTIME, np.sort(rng.integers(NOW - 86400, NOW, 40))),
         (CANDIDATE, rng.integers(NOW - 86400, NOW, 30))],
        [(PROFILE, np.full(5, NOW - 200 * 86400)),
         (HISTORY, np.sort(rng.integers(NOW - 200 * 86400, NOW - 86400, 300)))],
        [(HISTORY, np.sort(rng.integers(NOW - 100 * 86400, NOW, 200)))],
    ]
    wl = make_custom(reqs, heads=2, d_head=64, dtype="bf16", seed=31, delay=0)
    wl.q[:, :, :8] += 2.0
    offs = wl.req_offsets
    hot = []
    for r in range(offs.shape[0] - 1):
        hist = np.nonzero(wl.seg_kind[offs[r]:offs[r + 1]] == HISTORY)[0]
        j = int(offs[r] + hist[int(0.6 * hist.shape[0])])
        wl.k[j, :, :8] = 40.0
        hot.append(j)
    from rk_workloads import bf16_round
    wl.q = bf16_round(wl.q.astype(np.float32))
    wl.k = bf16_round(wl.k.astype(np.float32))
    plan, o, lse = _run(rk, wl, rope=rope)
    ref, ref_lse = _oracle_full(wl, rope=rope)
    _check(wl, o, ref)
    # The rows that see a hot key are that key's value row to bf16 precision.
    sees = np.zeros(wl.total_tokens, bool)
    for r, j in enumerate(hot):
        L = int(offs[r + 1] - offs[r])
        rows = oracle.visible_rows(wl.seg_kind[offs[r]:offs[r + 1]],
                                   wl.timestamps[offs[r]:offs[r + 1]], np.arange(L),
                                   delay=wl.delay, window=wl.window,
                                   static_bidirectional=wl.static_bidirectional)
        for p, vis in enumerate(rows):
            if vis[j - offs[r]]:
                sees[offs[r] + p] = True
                assert np.abs(o[offs[r] + p] - wl.v[j]).max() <= BF16_MAX_ABS
    assert sees.sum() > 300
    # lse: the bf16 query carries up to 2^-9 relative rounding into a score
    # of ~80, so the bound here grows with |lse|.
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.all(np.abs(lse[fin] - ref_lse[fin]) <= 2e-2 + 2.0 ** -7 * np.abs(ref_lse[fin]))


@pytest.mark.parametrize("rope", [True, False], ids=["rope", "norope"])
def test_attention_scores_far_below_zero(rk, rope):
    """Every score of every row lies about 200 log2 units below zero
    (dimensions 0..7: query +12, key -12, the four lowest-frequency RoPE
    pairs, which turn by < 1e-3 rad over the span).  exp2 of such a score
    underflows fp32, so the kernel must move each row's reference down to
    its first visible tile's max; softmax is shift invariant, so the output
    is an ordinary weighted mean of V and the LSE is about -144."""
    rng = np.random.default_rng(47)
    reqs = [
        [(HISTORY, np.sort(rng.integers(NOW - 300 * 86400, NOW - 86400, 700))),
         (REALTIME, np.sort(rng.integers(NOW - 86400, NOW, 40))),
         (CANDIDATE, rng.integers(NOW - 86400, NOW, 30))],
        [(PROFILE, np.full(5, NOW - 200 * 86400)),
         (HISTORY, np.sort(rng.integers(NOW - 200 * 86400, NOW - 86400, 300)))],
    ]
    wl = make_custom(reqs, heads=2, d_head=64, dtype="bf16", seed=47, delay=3600)
    wl.q[:, :, :8] = 12.0
    wl.k[:, :, :8] = -12.0
    from rk_workloads import bf16_round
    wl.q = bf16_round(wl.q.astype(np.float32))
    wl.k = bf16_round(wl.k.astype(np.float32))
    plan, o, lse = _run(rk, wl, rope=rope)
    ref, ref_lse = _oracle_full(wl, rope=rope)
    _check(wl, o, ref)
    fin = np.isfinite(ref_lse)
    assert fin.sum() > 0.9 * fin.size
    assert np.all(ref_lse[fin] < -100)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.all(np.abs(lse[fin] - ref_lse[fin]) <= 2e-2 + 2.0 ** -7 * np.abs(ref_lse[fin]))


def _check_blocks(sched, sizes_of, group_of):
    """Blocks of each XCD queue (slot s runs on queue s % 8) of a schedule;
    returns how many blocks hold more than one group."""
    multi = 0
    for q in range(8):
        items = sched[q::8]
        items = items[items >= 0]
        groups = group_of(items).tolist()
        sizes = sizes_of(items).tolist()
        total = {g: groups.count(g) for g in set(groups)}
        left = dict(total)
        last = {}
        i = 0
        while i < len(items):
            # a block: its groups start in its first slots
            block = []
            while i < len(items) and groups[i] not in last:
                block.append(groups[i])
                last[groups[i]] = sizes[i]
                left[groups[i]] -= 1
                i += 1
            n = len(block)
            while i < len(items) and any(left[g] for g in block):
                g = groups[i]
                assert g in block, f"queue {q}: group {g} starts inside a block"
                assert sizes[i] <= last[g], f"queue {q}: a group's item sizes grow"
                last[g] = sizes[i]
                left[g] -= 1
                i += 1
            size = sum(total[g] for g in block)
            assert size <= 96 or n == 1, (q, size, n)
            multi += n > 1
    return multi


@pytest.mark.parametrize("cfg", [2, 4, 5])
def test_schedule_order(rk, cfg):
    """Launch order inside each XCD queue, for the forward's query-tile
    schedule and the backward's key-block schedule: the queue is a sequence
    of blocks, each holding the items of whole (request, head) groups, at
    most 96 items unless it is one group; every group of a block starts in
    the block's first slots (its largest item), and each group's items come
    in non-increasing size (non-empty tiles of the query tile, or of the key
    block)."""
    wl = make_config(cfg, with_qkv=False)
    _say(f"[gpu] schedule order workload {cfg}")
    batch = rk.Batch.from_workload(wl)
    plan = rk.Plan(batch, delay=wl.delay, window=wl.window,
                   static_bidirectional=wl.static_bidirectional, num_heads=wl.heads,
                   global_tail=wl.global_tail, backward=True)
    torch.cuda.synchronize()
    H = wl.heads
    nqts = [-(-(int(b) - int(a)) // 128) for a, b in zip(wl.req_offsets[:-1], wl.req_offsets[1:])]
    tile_req = np.repeat(np.arange(wl.num_requests), nqts)  # also each key block's request
    group_of = lambda items: tile_req[items // H] * H + items % H
    for name, sched, ptr in (("query tiles", plan.sched(), plan.qtile_ptr()),
                             ("key blocks", plan.ksched(), plan.kt_ptr())):
        nnz = np.diff(ptr.cpu().numpy().astype(np.int64))
        multi = _check_blocks(sched.cpu().numpy(), lambda items: nnz[items // H], group_of)
        if cfg in (2, 4):
            assert multi > 0, f"{name}: small groups expected to share blocks"
        else:
            assert multi == 0, f"{name}: groups of more than 96 items run alone"
    plan.close()
