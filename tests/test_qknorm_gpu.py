"""GPU parity of QK Norm (RMSNorm of Q and K rows before time RoPE) through
the C ABI against the CPU fp64 oracle.

* rk_qk_norm_rope (norm, then rotation by t - anchor, or norm only):
  fp32 within 1e-5, bf16 within one bf16 rounding (2^-8 relative to the
  row's magnitude); vector and scalar paths; every d it supports.
* Attention with qk_norm: MFMA (bf16, d = 64 and 128) and plain kernels (fp32 and
  bf16, d = 32, 64, 128), K normalised by the attention's own pass or
  prepared by rk_qk_norm_rope (RK_ATTN_K_PREROTATED), against the oracle;
  fp32 within 1e-4 max-abs, bf16 within 2e-2 max-abs and 1e-2 relative L2.
* The serving call with QK Norm: candidate keys normalised and rotated into
  a key cache by kind, the history's prepared once, a candidates-only plan;
  candidate rows equal the full call's bit for bit (whole items) or within
  the split bound (split items) and match the oracle.
* A full-size workload on sampled rows.  (The backward through QK Norm is
  checked with the other backward tests.)
"""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from rk_workloads import make_config, make_custom, random_layout  # noqa: E402

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


def _t_rel(wl):
    return wl.timestamps - np.repeat(wl.anchors, np.diff(wl.req_offsets))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_qk_norm_rope_pass(rk, dtype, d):
    rng = np.random.default_rng(d)
    wl = make_custom(random_layout(rng, 4, 300), heads=3, d_head=d, dtype=dtype, seed=d)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.from_numpy(rng.uniform(0.5, 1.5, d).astype(np.float32)).cuda()
    batch = rk.Batch.from_workload(wl)
    x = torch.from_numpy(wl.q * 3.0).cuda().to(tdt)  # rows of RMS near 3
    x_np = x.float().cpu().numpy().astype(np.float64)
    for gamma in (None, g):
        for rope in (None, _rope(wl)):
            for strided in (False, True):
                _say(f"[gpu] qk_norm_rope {dtype} d={d} gamma={gamma is not None} "
                     f"rope={rope is not None} strided={strided}")
                src = x
                if strided:  # odd token stride: the one-pair-per-thread path
                    big = torch.zeros((x.shape[0], x.shape[1] * d + 1), dtype=tdt, device="cuda")
                    big[:, :x.shape[1] * d] = x.reshape(x.shape[0], -1)
                    src = big[:, :x.shape[1] * d].view(x.shape[0], x.shape[1], d)
                y = rk.rk_qk_norm_rope(batch, src, eps=1e-6, gamma=gamma, rope=rope)
                torch.cuda.synchronize()
                ref = oracle.qk_rmsnorm(x_np, None if gamma is None else
                                        gamma.cpu().numpy().astype(np.float64), 1e-6)
                if rope is not None:
                    ref = oracle.time_rope(ref, _t_rel(wl), **rope)
                got = y.float().cpu().numpy()
                tol = 1e-5 if dtype == "f32" else 2.0 ** -8
                scale = np.maximum(np.abs(ref).max(axis=-1, keepdims=True), 1.0)
                assert np.all(np.abs(got - ref) <= tol * scale), np.abs(got - ref).max()


CASES = [("bf16", 64, False), ("f32", 32, True), ("f32", 64, True), ("f32", 128, True),
         ("bf16", 32, True), ("bf16", 128, True)]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-d{c[1]}-{'ref' if c[2] else 'mfma'}"
                                             for c in CASES])
def test_attention_with_qk_norm(rk, case):
    dtype, d, reference = case
    rng = np.random.default_rng(d + 1)
    wl = make_custom(random_layout(rng, 4, 420), heads=2, d_head=d, dtype=dtype, seed=d + 1,
                     delay=600, window=150, global_tail=30)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gq = rng.uniform(0.5, 1.5, d).astype(np.float32)
    gk = rng.uniform(0.5, 1.5, d).astype(np.float32)
    gq_t, gk_t = torch.from_numpy(gq).cuda(), torch.from_numpy(gk).cuda()
    batch = rk.Batch.from_workload(wl)
    plan = rk.Plan(batch, delay=wl.delay, window=wl.window, global_tail=wl.global_tail,
                   num_heads=wl.heads)
    # Q and K scaled by 2 (the norm removes it); V as drawn, so that |O|
    # stays well below 8, where the output's bf16 half-ulp (2^-9 |O|) alone
    # would use most of the 2e-2 bound
    q, k = (torch.from_numpy(a * 2.0).cuda().to(tdt) for a in (wl.q, wl.k))
    v = torch.from_numpy(wl.v).cuda().to(tdt)
    qn, kn, vn = (t.float().cpu().numpy().astype(np.float64) for t in (q, k, v))
    for rope in (_rope(wl), None):
        for pre in (False, True):
            _say(f"[gpu] attention qk_norm {case} rope={rope is not None} k_prepared={pre}")
            kk = k
            if pre:
                kk = rk.rk_qk_norm_rope(batch, k, eps=1e-5, gamma=gk_t, rope=rope)
            o, _ = rk.rk_masked_attn_fwd(plan, q, kk, v, rope=rope, reference=reference,
                                         k_prerotated=pre,
                                         qk_norm=dict(eps=1e-5, gamma_q=gq_t, gamma_k=gk_t))
            torch.cuda.synchronize()
            ref, _ = oracle.attention_forward(
                wl.req_offsets, wl.seg_kind, wl.timestamps, qn, kn, vn, delay=wl.delay,
                window=wl.window, static_bidirectional=False, rope=rope,
                rope_times=_t_rel(wl) if rope is not None else None, global_tail=wl.global_tail,
                qk_norm=dict(eps=1e-5, gamma_q=gq.astype(np.float64),
                             gamma_k=gk.astype(np.float64)))
            got = o.float().cpu().numpy().astype(np.float64)
            err = np.abs(got - ref).max()
            if dtype == "f32":
                assert err <= 1e-4, err
            else:
                rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
                assert err <= 2e-2 and rel <= 1e-2, (err, rel)


def test_qk_norm_workload_sampled_rows(rk):
    """The MTGR-shaped workload (16 x 3332 tokens, H = 8) with QK Norm, time
    RoPE and the benchmark's launch form, on sampled rows."""
    wl = make_config(4)
    rng = np.random.default_rng(4)
    gq = rng.uniform(0.5, 1.5, 64).astype(np.float32)
    gk = rng.uniform(0.5, 1.5, 64).astype(np.float32)
    batch = rk.Batch.from_workload(wl)
    plan = rk.Plan(batch, static_bidirectional=True, num_heads=wl.heads)
    q, k, v = (torch.from_numpy(a).cuda().to(torch.bfloat16) for a in (wl.q, wl.k, wl.v))
    o, _ = rk.rk_masked_attn_fwd(plan, q, k, v, rope=_rope(wl),
                                 qk_norm=dict(eps=1e-6, gamma_q=torch.from_numpy(gq).cuda(),
                                              gamma_k=torch.from_numpy(gk).cuda()))
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([rng.choice(wl.total_tokens, 60, replace=False),
                                     [0, wl.total_tokens - 1]]))
    qn = oracle.qk_rmsnorm(wl.q.astype(np.float64), gq, 1e-6)
    kn = oracle.qk_rmsnorm(wl.k.astype(np.float64), gk, 1e-6)
    got, ref = [], []
    for h in (0, wl.heads - 1):
        orow, _ = oracle.attention_rows(wl.req_offsets, wl.seg_kind, wl.timestamps, qn, kn, wl.v,
                                        toks, h, delay=0, window=0, static_bidirectional=True,
                                        rope=_rope(wl))
        got.append(o[toks, h].float().cpu().numpy())
        ref.append(orow)
    got, ref = np.concatenate(got), np.concatenate(ref)
    err = np.abs(got - ref).max()
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert err <= 2e-2 and rel <= 1e-2, (err, rel)


@pytest.mark.parametrize("heads,reqs_seed", [(2, 71), (8, 72)])
def test_qk_norm_serving_call(rk, heads, reqs_seed):
    from rk_workloads import CANDIDATE, HISTORY, PROFILE, REALTIME, NOW
    rng = np.random.default_rng(reqs_seed)
    reqs = []
    for n in (1500, 700, 300):
        hist = np.sort(rng.integers(NOW - 10**6, NOW - 3600, n)).astype(np.int64)
        reqs.append([(PROFILE, np.full(8, NOW, np.int64)), (HISTORY, hist),
                     (REALTIME, np.sort(rng.integers(NOW - 3600, NOW, 20)).astype(np.int64)),
                     (CANDIDATE, np.full(40, NOW, np.int64))])
    wl = make_custom(reqs, heads=heads, d_head=64, dtype="bf16", seed=reqs_seed, delay=1800)
    gq = rng.uniform(0.5, 1.5, 64).astype(np.float32)
    gk = rng.uniform(0.5, 1.5, 64).astype(np.float32)
    gq_t, gk_t = torch.from_numpy(gq).cuda(), torch.from_numpy(gk).cuda()
    norm = dict(eps=1e-5, gamma_q=gq_t, gamma_k=gk_t)
    batch = rk.Batch.from_workload(wl)
    q, k = (torch.from_numpy(a * 2.0).cuda().to(torch.bfloat16) for a in (wl.q, wl.k))
    v = torch.from_numpy(wl.v).cuda().to(torch.bfloat16)
    kw = dict(delay=wl.delay, num_heads=wl.heads)
    full_plan = rk.Plan(batch, **kw)
    cand_plan = rk.Plan(batch, candidates_only=True, **kw)
    _say(f"[gpu] qk-norm serving call heads={heads}")
    # the history's keys prepared once into the cache, the candidates' per call
    cache = torch.empty_like(k)
    rk.rk_qk_norm_rope(batch, k, eps=1e-5, gamma=gk_t, rope=_rope(wl), out=cache,
                       kinds=(PROFILE, HISTORY, REALTIME))
    rk.rk_qk_norm_rope(batch, k, eps=1e-5, gamma=gk_t, rope=_rope(wl), out=cache,
                       kinds=(CANDIDATE,))
    o_full, _ = rk.rk_masked_attn_fwd(full_plan, q, k, v, rope=_rope(wl), qk_norm=norm)
    o_c = torch.zeros_like(o_full)
    rk.rk_masked_attn_fwd(cand_plan, q, cache, v, out=o_c, rope=_rope(wl), qk_norm=norm,
                          k_prerotated=True)
    torch.cuda.synchronize()
    cand = np.nonzero(wl.seg_kind == CANDIDATE)[0]
    st = cand_plan.stats()
    got, full = o_c[torch.from_numpy(cand).cuda()], o_full[torch.from_numpy(cand).cuda()]
    if st["split_items"] == 0:
        assert torch.equal(got.view(torch.int16), full.view(torch.int16))
    else:
        err = (got.float() - full.float()).abs().max().item()
        assert err <= 2e-2, err
    qn, kn, vn = (t.float().cpu().numpy().astype(np.float64) for t in (q, k, v))
    ref, _ = oracle.attention_forward(
        wl.req_offsets, wl.seg_kind, wl.timestamps, qn, kn, vn, delay=wl.delay, window=0,
        static_bidirectional=False, rope=_rope(wl), rope_times=_t_rel(wl),
        qk_norm=dict(eps=1e-5, gamma_q=gq.astype(np.float64), gamma_k=gk.astype(np.float64)))
    ref = ref[cand]
    o_np = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(o_np - ref).max()
    assert err <= 2e-2, err
    assert np.linalg.norm(o_np - ref) <= 1e-2 * np.linalg.norm(ref)
    full_plan.close()
    cand_plan.close()
