"""GPU parity of the masked-attention backward (through the C ABI) against
the CPU fp64 oracle.

* Key-major tables of a backward plan: for every block of 128 keys, the
  ascending list of query tiles with a visible pair and their PARTIAL bits
  are bit-exact against the oracle's tile plan read by columns; the
  key-major schedule covers every (key block, head) once; the query-major tables are
  the same as those of a forward-only plan.
* Gradients: dQ, dK, dV against the oracle's chain-rule gradients on the
  same inputs (the GPU's own forward O and LSE feed its backward).  fp32:
  within 1e-4 max-abs.  bf16: relative L2 within 1e-2 and max-abs within
  2e-2 * max(1, max |reference|) (bf16 outputs round to 2^-9 relative, so a
  fixed absolute bound cannot hold for gradients above 4 in magnitude).
"""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from rk_workloads import (CANDIDATE, HISTORY, NOW, PROFILE, REALTIME, draw_grad,  # noqa: E402
                          make_config, make_custom, random_layout)

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
    _rk.lib()
    return m


def _rope(wl):
    return dict(phi_min=wl.phi_min, dt_max=wl.dt_max, base=wl.base)


def _dt(wl):
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def _plan(rk, wl, backward=True, batch=None):
    batch = batch or rk.Batch.from_workload(wl)
    plan = rk.Plan(batch, delay=wl.delay, window=wl.window,
                   static_bidirectional=wl.static_bidirectional, num_heads=wl.heads,
                   global_tail=wl.global_tail, backward=backward)
    return batch, plan


def _key_major_ref(wl):
    """Oracle tile plan read by columns over key blocks of 128 keys (k-tiles
    2 kb and 2 kb + 1): per global key block, ascending query tiles with a
    visible pair in either k-tile, bit 31 set unless both k-tiles exist and
    are FULL."""
    ptr, words = [0], []
    for r in range(wl.num_requests):
        a, b = wl.request(r)
        if b == a:
            continue
        cnt, cls = oracle.tile_plan_request(wl.seg_kind[a:b], wl.timestamps[a:b], delay=wl.delay,
                                            window=wl.window,
                                            static_bidirectional=wl.static_bidirectional,
                                            global_tail=wl.global_tail)
        nkt = cnt.shape[1]
        for kb in range(-(-(b - a) // 128)):
            cols = [c for c in (2 * kb, 2 * kb + 1) if c < nkt]
            qts = np.nonzero(cnt[:, cols].sum(axis=1))[0]
            for qt in qts:
                full = len(cols) == 2 and all(cls[qt, c] == oracle.FULL for c in cols)
                words.append(int(qt) | (0 if full else (1 << 31)))
            ptr.append(ptr[-1] + qts.shape[0])
    w = np.array(words, dtype=np.uint32).view(np.int32) if words else np.zeros(0, np.int32)
    return np.array(ptr, np.int64), w


def _check_key_major(rk, wl):
    batch, plan = _plan(rk, wl)
    _, fplan = _plan(rk, wl, backward=False, batch=batch)
    torch.cuda.synchronize()
    assert plan.stats()["device_errors"] == 0
    ptr_ref, words_ref = _key_major_ref(wl)
    assert np.array_equal(plan.kt_ptr().cpu().numpy().astype(np.int64), ptr_ref)
    assert np.array_equal(plan.qtile_word().cpu().numpy(), words_ref)
    ks = plan.ksched().cpu().numpy()
    items = np.sort(ks[ks >= 0])
    assert np.array_equal(items, np.arange(plan.num_kblocks * wl.heads))
    # the query-major tables are those of a forward-only plan
    for f in ("tile_class", "tile_count", "qtile_ptr", "ktile_idx", "sched", "row_desc"):
        assert torch.equal(getattr(plan, f)(), getattr(fplan, f)()), f
    assert fplan.kt_ptr() is None


def test_key_major_tables_random_layouts(rk):
    for seed in range(6):
        rng = np.random.default_rng(100 + seed)
        reqs = random_layout(rng, 5, 700)
        for bidir, delay, window, G in ((False, 3600, 0, 0), (True, 0, 0, 0), (False, 0, 130, 70),
                                        (False, 60, 200, 0)):
            _say(f"[gpu] key-major seed={seed} bidir={bidir} delay={delay} window={window} G={G}")
            wl = make_custom(reqs, heads=3, d_head=64, seed=seed, delay=delay, window=window,
                             static_bidirectional=bidir, global_tail=G, with_qkv=False)
            _check_key_major(rk, wl)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_key_major_tables_workloads(rk, cfg):
    _say(f"[gpu] key-major workload {cfg}")
    _check_key_major(rk, make_config(cfg, with_qkv=False))


def _grads_gpu(rk, wl, rope, reference=False, k_prerotated=False, strided=False):
    batch, plan = _plan(rk, wl)
    dt = _dt(wl)
    q, k, v = (torch.from_numpy(x).to("cuda").to(dt) for x in (wl.q, wl.k, wl.v))
    do = torch.from_numpy(draw_grad(wl)).to("cuda").to(dt)
    if strided:
        # [T, H, d] views with padded token and head strides
        def pad(x):
            T, H, d = x.shape
            big = torch.zeros((T, H + 1, d + 8), dtype=x.dtype, device=x.device)
            big[:, :H, :d] = x
            return big[:, :H, :d]
        q, k, v, do = pad(q), pad(k), pad(v), pad(do)
    rp = _rope(wl) if rope else None
    k_in = k
    if k_prerotated:
        k_in = rk.rk_time_rope(batch, k, **rp)
    o, lse = rk.rk_masked_attn_fwd(plan, q, k_in, v, rope=rp, want_lse=True,
                                   reference=reference, k_prerotated=k_prerotated)
    dq, dk, dv = rk.rk_masked_attn_bwd(plan, q, k_in, v, o, lse, do, rope=rp,
                                       reference=reference, k_prerotated=k_prerotated)
    torch.cuda.synchronize()
    f = lambda x: x.float().cpu().numpy().astype(np.float64)
    return f(dq), f(dk), f(dv), draw_grad(wl)


def _check_grad(wl, got, ref, what):
    err = np.abs(got - ref)
    if wl.dtype == "f32":
        assert err.max() <= F32_TOL, f"{what}: max abs {err.max()}"
    else:
        rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
        bound = BF16_MAX_ABS * max(1.0, float(np.abs(ref).max()))
        assert rel <= BF16_REL_L2, f"{what}: rel L2 {rel}"
        assert err.max() <= bound, f"{what}: max abs {err.max()} > {bound}"


def _oracle_grads(wl, do, rope, k_prerotated=False):
    """Oracle gradients with respect to the tensors the GPU call was given:
    unrotated q, k, v; with k_prerotated, k is passed rotated by (t - anchor),
    so dk is the gradient with respect to that rotated key."""
    q, k, v = (x.astype(np.float64) for x in (wl.q, wl.k, wl.v))
    margs = dict(delay=wl.delay, window=wl.window, static_bidirectional=wl.static_bidirectional,
                 global_tail=wl.global_tail)
    if not k_prerotated:
        return oracle.attention_backward(wl.req_offsets, wl.seg_kind, wl.timestamps, q, k, v,
                                         do.astype(np.float64),
                                         rope=_rope(wl) if rope else None, **margs)
    t_rel = wl.timestamps - np.repeat(wl.anchors, np.diff(wl.req_offsets))
    qr = oracle.time_rope(q, t_rel, **_rope(wl))
    kr = oracle.time_rope(k, t_rel, **_rope(wl))
    dq_r, dk_r, dv = oracle.attention_backward(wl.req_offsets, wl.seg_kind, wl.timestamps, qr,
                                               kr, v, do.astype(np.float64), **margs)
    return oracle.time_rope_transpose(dq_r, t_rel, **_rope(wl)), dk_r, dv


CASES = [
    # (dtype, d, reference, bidir, delay, window, G)
    ("f32", 32, True, False, 3600, 0, 0),
    ("f32", 64, True, True, 0, 0, 0),
    ("f32", 128, True, False, 0, 100, 0),
    ("bf16", 32, True, False, 60, 0, 0),
    ("bf16", 64, True, False, 0, 90, 40),
    ("bf16", 128, True, True, 0, 0, 0),
    ("bf16", 64, False, False, 3600, 0, 0),
    ("bf16", 64, False, True, 0, 0, 0),
    ("bf16", 64, False, False, 0, 150, 64),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-d{c[1]}-{'ref' if c[2] else 'mfma'}-b{int(c[3])}-D{c[4]}-W{c[5]}-G{c[6]}" for c in CASES])
def test_backward_matches_oracle(rk, case):
    dtype, d, reference, bidir, delay, window, G = case
    rng = np.random.default_rng(d + delay + window)
    reqs = random_layout(rng, 4, 460)
    for rope in (True, False):
        _say(f"[gpu] backward {case} rope={rope}")
        wl = make_custom(reqs, heads=2, d_head=d, dtype=dtype, seed=d + window, delay=delay,
                         window=window, static_bidirectional=bidir, global_tail=G)
        dq, dk, dv, do = _grads_gpu(rk, wl, rope, reference=reference)
        rq, rk_, rv = _oracle_grads(wl, do, rope)
        _check_grad(wl, dq, rq, "dq")
        _check_grad(wl, dk, rk_, "dk")
        _check_grad(wl, dv, rv, "dv")


@pytest.mark.parametrize("reference", [True, False])
def test_backward_strided_and_prerotated(rk, reference):
    rng = np.random.default_rng(77)
    reqs = random_layout(rng, 3, 400, allow_empty=False)
    wl = make_custom(reqs, heads=3, d_head=64, dtype="bf16", seed=77, delay=600, window=0)
    for strided, pre in ((True, False), (False, True)):
        _say(f"[gpu] backward strided={strided} k_prerotated={pre} reference={reference}")
        dq, dk, dv, do = _grads_gpu(rk, wl, True, reference=reference, k_prerotated=pre,
                                    strided=strided)
        rq, rk_, rv = _oracle_grads(wl, do, True, k_prerotated=pre)
        _check_grad(wl, dq, rq, "dq")
        _check_grad(wl, dk, rk_, "dk")
        _check_grad(wl, dv, rv, "dv")


def test_backward_empty_rows_and_unseen_keys_are_zero(rk):
    """Rows that see nothing get dQ = 0 and keys nobody sees get dK = dV = 0,
    exactly, also where the output buffers held other values."""
    hist = np.sort(np.random.default_rng(5).integers(NOW - 6 * 3600, NOW, size=300))
    wl = make_custom([[(HISTORY, hist)]], heads=2, d_head=64, dtype="bf16", seed=5, delay=3600)
    batch, plan = _plan(rk, wl)
    q, k, v = (torch.from_numpy(x).to("cuda").to(torch.bfloat16) for x in (wl.q, wl.k, wl.v))
    do = torch.from_numpy(draw_grad(wl)).to("cuda").to(torch.bfloat16)
    o, lse = rk.rk_masked_attn_fwd(plan, q, k, v, rope=_rope(wl), want_lse=True)
    for reference in (True, False):
        dq, dk, dv = (torch.full_like(q, 7.0) for _ in range(3))
        rk.rk_masked_attn_bwd(plan, q, k, v, o, lse, do, rope=_rope(wl), dq=dq, dk=dk, dv=dv,
                              reference=reference)
        torch.cuda.synchronize()
        vis = oracle.visibility(wl.seg_kind, wl.timestamps, delay=wl.delay, window=0,
                                static_bidirectional=False)
        empty = torch.from_numpy(~vis.any(axis=1)).cuda()
        unseen = torch.from_numpy(~vis.any(axis=0)).cuda()
        assert empty.sum() > 0 and unseen.sum() > 0
        assert torch.all(dq[empty] == 0) and torch.all(dk[unseen] == 0)
        assert torch.all(dv[unseen] == 0)
        assert not torch.any(dq == 7.0) and not torch.any(dk == 7.0)


def test_backward_deterministic(rk):
    wl = make_config(2)
    wl = make_custom([[(HISTORY, wl.timestamps[:1024])], [(HISTORY, wl.timestamps[1024:1800])]],
                     heads=4, d_head=64, dtype="bf16", seed=3, delay=3600)
    a = _grads_gpu(rk, wl, True)
    b = _grads_gpu(rk, wl, True)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)


def test_backward_rejects_forward_only_plan(rk):
    from masked_attention_amd import _rk
    wl = make_custom([[(HISTORY, np.arange(NOW - 200, NOW, 2, dtype=np.int64))]], heads=1,
                     d_head=64, dtype="bf16", seed=1)
    batch, plan = _plan(rk, wl, backward=False)
    q = torch.from_numpy(wl.q).cuda().to(torch.bfloat16)
    o, lse = rk.rk_masked_attn_fwd(plan, q, q, q, want_lse=True)
    with pytest.raises(_rk.RkError) as e:
        rk.rk_masked_attn_bwd(plan, q, q, q, o, lse, q)
    assert e.value.status == _rk.RK_ERR_INVALID_ARG
    _, bplan = _plan(rk, wl, batch=batch)
    with pytest.raises(_rk.RkError) as e:
        rk.rk_masked_attn_bwd(bplan, q, q, q, o, None, q)
    assert e.value.status == _rk.RK_ERR_INVALID_ARG


def _sampled_positions(wl, cfg, r, rng):
    """Rows (dQ) and keys (dK, dV) of request r compared on a full-size
    workload: its first and last positions, random ones and candidates.
    On the TM20K shape the keys of requests other than the first are drawn
    from the last 1024 positions (the oracle then needs the statistics of
    those rows only)."""
    a, b = wl.request(r)
    L = b - a
    pick = lambda lo, n: rng.choice(np.arange(lo, L), size=min(n, L - lo), replace=False)
    rows = np.concatenate([[0, L - 1], pick(0, 6)])
    if cfg == 5 and r > 0:
        keys = np.concatenate([[L - 1], pick(max(0, L - 1024), 4)])
    else:
        keys = np.concatenate([[0, L - 1], pick(0, 6)])
    cand = np.nonzero(wl.seg_kind[a:b] == CANDIDATE)[0]
    if cand.shape[0]:
        rows = np.concatenate([rows, cand[:2], cand[-2:]])
        keys = np.concatenate([keys, cand[:2]])
    return np.unique(rows), np.unique(keys)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_backward_workloads(rk, cfg):
    """Full-size workloads in the launch configuration the backward benchmark
    times (backward plan; forward with fused RoPE and LSE; backward with
    RoPE).  The CADET-shaped workload (2) is compared in full; the others on
    sampled rows (dQ) and keys (dK, dV) of every request, each request on
    its own head (head r mod H), against the oracle's per-row / per-key
    gradients."""
    wl = make_config(cfg)
    _say(f"[gpu] backward workload {cfg}: T={wl.total_tokens} H={wl.heads}")
    batch, plan = _plan(rk, wl)
    q, k, v = (torch.from_numpy(x).to("cuda").to(torch.bfloat16) for x in (wl.q, wl.k, wl.v))
    do_np = draw_grad(wl)
    do = torch.from_numpy(do_np).to("cuda").to(torch.bfloat16)
    o, lse = rk.rk_masked_attn_fwd(plan, q, k, v, rope=_rope(wl), want_lse=True)
    dq, dk, dv = rk.rk_masked_attn_bwd(plan, q, k, v, o, lse, do, rope=_rope(wl))
    torch.cuda.synchronize()
    host = lambda x: x.float().cpu().numpy().astype(np.float64)
    if cfg == 2:
        rq, rk_, rv = oracle.attention_backward(
            wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q, wl.k, wl.v, do_np, delay=wl.delay,
            window=wl.window, static_bidirectional=wl.static_bidirectional, rope=_rope(wl))
        _check_grad(wl, host(dq), rq, "dq")
        _check_grad(wl, host(dk), rk_, "dk")
        _check_grad(wl, host(dv), rv, "dv")
        return
    rng = np.random.default_rng(cfg)
    dq_h, dk_h, dv_h = host(dq), host(dk), host(dv)
    got, ref = [], []
    for r in range(wl.num_requests):
        a, b = wl.request(r)
        h = r % wl.heads
        rows, keys = _sampled_positions(wl, cfg, r, rng)
        rq, rk_, rv = oracle.attention_backward_sampled(
            wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q, wl.k, wl.v, do_np, request=r,
            head=h, rows=rows, keys=keys, delay=wl.delay, window=wl.window,
            static_bidirectional=wl.static_bidirectional, rope=_rope(wl),
            global_tail=wl.global_tail)
        got += [dq_h[a + rows, h].ravel(), dk_h[a + keys, h].ravel(), dv_h[a + keys, h].ravel()]
        ref += [rq.ravel(), rk_.ravel(), rv.ravel()]
        if r % 8 == 7 or r == wl.num_requests - 1:
            _say(f"[gpu] backward workload {cfg}: requests up to {r} sampled")
    got, ref = np.concatenate(got), np.concatenate(ref)
    _check_grad(wl, got, ref, f"workload {cfg} sampled gradients")


def test_backward_tiny_fp32_workload_full(rk):
    """The fp32 workload (one request of 256 history + 16 candidates, H = 2,
    d = 32, one-hour delay, time RoPE) compared element by element."""
    wl = make_config(1)
    _say(f"[gpu] backward {wl.name}")
    dq, dk, dv, do = _grads_gpu(rk, wl, True)
    rq, rk_, rv = _oracle_grads(wl, do, True)
    _check_grad(wl, dq, rq, "dq")
    _check_grad(wl, dk, rk_, "dk")
    _check_grad(wl, dv, rv, "dv")


QKN_CASES = [
    # (dtype, d, reference, rope, gains)
    ("f32", 32, True, True, True),
    ("f32", 64, True, False, True),
    ("f32", 128, True, True, False),
    ("bf16", 64, True, True, True),
    ("bf16", 128, True, False, True),
    ("bf16", 64, False, True, True),
    ("bf16", 64, False, False, True),
    ("bf16", 64, False, True, False),
]


def _check_gain(dtype, got, ref, what):
    err = np.abs(got - ref)
    scale = max(1.0, float(np.abs(ref).max()))
    if dtype == "f32":
        assert err.max() <= 1e-4 * scale, f"{what}: max abs {err.max()} (scale {scale})"
    else:
        rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
        assert rel <= BF16_REL_L2 and err.max() <= BF16_MAX_ABS * scale, (what, rel, err.max())


@pytest.mark.parametrize("case", QKN_CASES, ids=[
    f"{c[0]}-d{c[1]}-{'ref' if c[2] else 'mfma'}-{'rope' if c[3] else 'norope'}-"
    f"{'gains' if c[4] else 'nogain'}" for c in QKN_CASES])
def test_backward_qk_norm_matches_oracle(rk, case):
    """Backward through QK Norm (RMSNorm of the Q and K rows before the
    rotation): dQ, dK, dV and the gains' gradients against the oracle's
    chain rule (attention backward at the normalised rows, then the norm's)."""
    dtype, d, reference, rope, gains = case
    _say(f"[gpu] backward qk-norm {case}")
    rng = np.random.default_rng(500 + d)
    wl = make_custom(random_layout(rng, 3, 400), heads=2, d_head=d, dtype=dtype, seed=11 + d,
                     delay=600, window=0)
    gq = rng.uniform(0.5, 1.5, d).astype(np.float32) if gains else None
    gk = rng.uniform(0.5, 1.5, d).astype(np.float32) if gains else None
    eps = 1e-6
    batch, plan = _plan(rk, wl)
    dt = _dt(wl)
    q, k, v = (torch.from_numpy(x).to("cuda").to(dt) for x in (wl.q, wl.k, wl.v))
    do_np = draw_grad(wl)
    do = torch.from_numpy(do_np).to("cuda").to(dt)
    tg = lambda g: torch.from_numpy(g).cuda() if g is not None else None
    norm = dict(eps=eps, gamma_q=tg(gq), gamma_k=tg(gk))
    rp = _rope(wl) if rope else None
    o, lse = rk.rk_masked_attn_fwd(plan, q, k, v, rope=rp, want_lse=True, reference=reference,
                                   qk_norm=norm)
    dq, dk, dv, dgq, dgk = rk.rk_masked_attn_bwd(plan, q, k, v, o, lse, do, rope=rp,
                                                 reference=reference, qk_norm=norm)
    torch.cuda.synchronize()
    q64, k64, v64 = (x.astype(np.float64) for x in (wl.q, wl.k, wl.v))
    g64 = lambda g: g.astype(np.float64) if g is not None else None
    rq, rk_, rv, rgq, rgk = oracle.attention_backward_qk_norm(
        wl.req_offsets, wl.seg_kind, wl.timestamps, q64, k64, v64, do_np.astype(np.float64),
        qk_norm=dict(eps=eps, gamma_q=g64(gq), gamma_k=g64(gk)), delay=wl.delay,
        window=wl.window, static_bidirectional=False, rope=rp)
    f = lambda x: x.float().cpu().numpy().astype(np.float64)
    _check_grad(wl, f(dq), rq, "dq")
    _check_grad(wl, f(dk), rk_, "dk")
    _check_grad(wl, f(dv), rv, "dv")
    if gains:
        _check_gain(dtype, dgq.cpu().numpy().astype(np.float64), rgq, "dgamma_q")
        _check_gain(dtype, dgk.cpu().numpy().astype(np.float64), rgk, "dgamma_k")
    else:
        assert dgq is None and dgk is None
    # the pass is deterministic
    again = rk.rk_masked_attn_bwd(plan, q, k, v, o, lse, do, rope=rp, reference=reference,
                                  qk_norm=norm)
    torch.cuda.synchronize()
    assert torch.equal(again[0], dq) and torch.equal(again[1], dk)
    if gains:
        assert torch.equal(again[3], dgq) and torch.equal(again[4], dgk)


def test_backward_qk_norm_workload_sampled(rk):
    """MTGR-shaped workload (16 x (32 + 3000 + 200 + 100), H = 8, static part
    bidirectional) with QK Norm and RoPE: sampled rows (dQ) and keys (dK, dV)
    of the first and last requests against the oracle at the normalised
    rows, taken back through the norm row by row."""
    wl = make_config(4)
    _say(f"[gpu] backward qk-norm sampled workload 4: T={wl.total_tokens} H={wl.heads}")
    rng = np.random.default_rng(44)
    d = wl.d_head
    gq = rng.uniform(0.5, 1.5, d).astype(np.float32)
    gk = rng.uniform(0.5, 1.5, d).astype(np.float32)
    eps = 1e-6
    batch, plan = _plan(rk, wl)
    q, k, v = (torch.from_numpy(x).to("cuda").to(torch.bfloat16) for x in (wl.q, wl.k, wl.v))
    do_np = draw_grad(wl)
    do = torch.from_numpy(do_np).to("cuda").to(torch.bfloat16)
    norm = dict(eps=eps, gamma_q=torch.from_numpy(gq).cuda(), gamma_k=torch.from_numpy(gk).cuda())
    o, lse = rk.rk_masked_attn_fwd(plan, q, k, v, rope=_rope(wl), want_lse=True, qk_norm=norm)
    dq, dk, dv, _, _ = rk.rk_masked_attn_bwd(plan, q, k, v, o, lse, do, rope=_rope(wl),
                                             qk_norm=norm)
    torch.cuda.synchronize()
    got, ref = [], []
    for r in (0, wl.num_requests - 1):
        a, b = wl.request(r)
        L = b - a
        pick = lambda n: np.unique(np.concatenate([[0, L - 1], rng.choice(L, size=n, replace=False)]))
        rows, keys = pick(20), pick(20)
        qn, kn = wl.q.astype(np.float64), wl.k.astype(np.float64)
        qn[a:b] = oracle.qk_rmsnorm(qn[a:b], gq.astype(np.float64), eps)
        kn[a:b] = oracle.qk_rmsnorm(kn[a:b], gk.astype(np.float64), eps)
        for h in (0, wl.heads - 1):
            gq_rows, gk_keys, rv = oracle.attention_backward_sampled(
                wl.req_offsets, wl.seg_kind, wl.timestamps, qn, kn, wl.v, do_np, request=r,
                head=h, rows=rows, keys=keys, delay=wl.delay, window=wl.window,
                static_bidirectional=wl.static_bidirectional, rope=_rope(wl))
            rq, _ = oracle.qk_rmsnorm_backward(wl.q[a + rows, h], gq.astype(np.float64), eps,
                                               gq_rows)
            rk_, _ = oracle.qk_rmsnorm_backward(wl.k[a + keys, h], gk.astype(np.float64), eps,
                                                gk_keys)
            f = lambda x, idx: x[a + idx, h].float().cpu().numpy().astype(np.float64)
            got += [f(dq, rows).ravel(), f(dk, keys).ravel(), f(dv, keys).ravel()]
            ref += [rq.ravel(), rk_.ravel(), rv.ravel()]
    _check_grad(wl, np.concatenate(got), np.concatenate(ref), "workload 4 qk-norm sampled")


def test_backward_qk_norm_rejections(rk):
    """QK Norm with a pre-rotated K, and a gain without its gradient
    pointer, are invalid arguments."""
    import ctypes as C

    from masked_attention_amd import _rk
    from masked_attention_amd.binding import _bwd_args, qk_norm_params
    wl = make_custom([[(HISTORY, np.arange(NOW - 900, NOW, 3, dtype=np.int64))]], heads=1,
                     d_head=64, dtype="bf16", seed=3)
    batch, plan = _plan(rk, wl)
    q = torch.from_numpy(wl.q).cuda().to(torch.bfloat16)
    lse = torch.zeros((1, wl.total_tokens), dtype=torch.float32, device="cuda")
    g = torch.ones(64, dtype=torch.float32, device="cuda")
    with pytest.raises(_rk.RkError) as e:
        rk.rk_masked_attn_bwd(plan, q, q, q, q, lse, q, rope=_rope(wl), k_prerotated=True,
                              qk_norm=dict(eps=1e-6))
    assert e.value.status == _rk.RK_ERR_INVALID_ARG
    out = [torch.empty_like(q) for _ in range(3)]
    a = _bwd_args(q, q, q, q, q, lse, *out, 0.0, None, False, False, None)
    nq = qk_norm_params(1e-6, gamma_q=g)
    a.qk_norm = C.cast(C.pointer(nq), C.c_void_p)
    assert _rk.lib().rk_masked_attn_bwd(plan.handle, C.byref(a), None) == _rk.RK_ERR_INVALID_ARG
