"""Degenerate batches through every entry point (GPU, through the C ABI).

* A batch with no tokens (two empty requests) and a batch with no requests:
  plans (forward, backward, candidates-only) build with no work, the
  rotation, the forward (MFMA and plain kernels, with LSE), the backward
  (with QK Norm: the gains' gradients are exactly zero) and the pointwise
  form all succeed and write nothing.
* Requests of one token, alone and next to longer ones: forward, backward
  and pointwise outputs against the oracle (a one-token request sees only
  itself: O = V, LSE = scale q.k and dV = dO up to one bf16 rounding).
"""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from rk_workloads import CANDIDATE, HISTORY, NOW, make_custom  # noqa: E402

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


def _rope(wl):
    return dict(phi_min=wl.phi_min, dt_max=wl.dt_max, base=wl.base)


@pytest.mark.parametrize("layout", [[[], []], []], ids=["empty-requests", "no-requests"])
def test_batch_without_tokens(rk, layout):
    _say(f"[gpu] degenerate batch {len(layout)} requests, no tokens")
    wl = make_custom(layout, heads=2, d_head=64, dtype="bf16", seed=1)
    assert wl.total_tokens == 0
    batch = rk.Batch.from_workload(wl)
    q = torch.zeros((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    rope = _rope(wl)
    for kw in (dict(), dict(backward=True), dict(candidates_only=True)):
        plan = rk.Plan(batch, num_heads=2, **kw)
        torch.cuda.synchronize()
        st = plan.stats()
        assert st["device_errors"] == 0 and st["visible_pairs"] == 0
        for reference in (False, True):
            o, lse = rk.rk_masked_attn_fwd(plan, q, q, q, rope=rope, want_lse=True,
                                           reference=reference)
            assert o.shape == (0, 2, 64) and lse.shape == (2, 0)
        if not kw.get("candidates_only"):
            o = rk.rk_pointwise_attn_fwd(plan, q, q, q, scale=0.125)
            assert o.shape == (0, 2, 64)
        if kw.get("backward"):
            lse = torch.zeros((2, 0), dtype=torch.float32, device="cuda")
            g = torch.ones(64, dtype=torch.float32, device="cuda")
            for reference in (False, True):
                dq, dk, dv, dgq, dgk = rk.rk_masked_attn_bwd(
                    plan, q, q, q, q, lse, q, rope=rope, reference=reference,
                    qk_norm=dict(eps=1e-6, gamma_q=g, gamma_k=g))
                torch.cuda.synchronize()
                assert dq.shape == (0, 2, 64)
                assert torch.equal(dgq, torch.zeros_like(dgq))
                assert torch.equal(dgk, torch.zeros_like(dgk))
        plan.close()
    out = rk.rk_time_rope(batch, q, **rope)
    torch.cuda.synchronize()
    assert out.shape == (0, 2, 64)


def test_one_token_requests(rk):
    """One-token requests (a lone history token, a lone candidate) among
    longer ones: forward, backward and pointwise against the oracle."""
    rng = np.random.default_rng(3)
    hist = np.sort(rng.integers(NOW - 10**6, NOW - 60, 200)).astype(np.int64)
    layout = [[(HISTORY, np.array([NOW - 100], np.int64))],
              [(HISTORY, hist), (CANDIDATE, np.full(3, NOW, np.int64))],
              [(CANDIDATE, np.array([NOW], np.int64))],
              [(HISTORY, hist[:129])]]
    wl = make_custom(layout, heads=2, d_head=64, dtype="bf16", seed=4)
    batch = rk.Batch.from_workload(wl)
    plan = rk.Plan(batch, num_heads=2, backward=True)
    q, k, v = (torch.from_numpy(x).cuda().to(torch.bfloat16) for x in (wl.q, wl.k, wl.v))
    rope = _rope(wl)
    q64, k64, v64 = (x.astype(np.float64) for x in (wl.q, wl.k, wl.v))
    margs = dict(delay=0, window=0, static_bidirectional=False)
    ro, rl = oracle.attention_forward(wl.req_offsets, wl.seg_kind, wl.timestamps, q64, k64, v64,
                                      rope=rope, **margs)
    do_np = rng.standard_normal(wl.q.shape).astype(np.float32)
    do = torch.from_numpy(do_np).cuda().to(torch.bfloat16)
    do64 = do.float().cpu().numpy().astype(np.float64)
    rq, rk_, rv = oracle.attention_backward(wl.req_offsets, wl.seg_kind, wl.timestamps, q64, k64,
                                            v64, do64, rope=rope, **margs)
    lone = [int(wl.req_offsets[0]), int(wl.req_offsets[2])]
    for reference in (False, True):
        _say(f"[gpu] one-token requests reference={reference}")
        o, lse = rk.rk_masked_attn_fwd(plan, q, k, v, rope=rope, want_lse=True,
                                       reference=reference)
        dq, dk, dv = rk.rk_masked_attn_bwd(plan, q, k, v, o, lse, do, rope=rope,
                                           reference=reference)
        torch.cuda.synchronize()
        f = lambda x: x.float().cpu().numpy().astype(np.float64)
        got_o = f(o)
        assert np.abs(got_o - ro).max() <= 2e-2 * max(1.0, np.abs(ro).max())
        assert np.allclose(lse.cpu().numpy(), rl, atol=2e-2, rtol=1e-2)
        for got, ref in ((f(dq), rq), (f(dk), rk_), (f(dv), rv)):
            err = np.abs(got - ref).max()
            assert err <= 2e-2 * max(1.0, np.abs(ref).max()), err
        # a lone token sees only itself: O = V and dV = dO up to one bf16
        # rounding (P is rounded to bf16 for the product, its sum is not)
        for t in lone:
            assert np.allclose(got_o[t], wl.v[t], rtol=2 ** -7, atol=1e-6)
            assert np.allclose(f(dv)[t], do64[t], rtol=2 ** -7, atol=1e-6)
    po = rk.rk_pointwise_attn_fwd(plan, q, k, v, scale=0.125)
    torch.cuda.synchronize()
    pref = oracle.pointwise_attention_forward(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q,
                                              wl.k, wl.v, scale=0.125, **margs)
    got = po.float().cpu().numpy().astype(np.float64)
    assert np.abs(got - pref).max() <= 2e-2 * max(1.0, np.abs(pref).max())
    plan.close()
