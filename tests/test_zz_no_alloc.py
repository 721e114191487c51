"""GPU test of rk_masked_attn_fwd_noalloc (the forward for callers that
cannot allocate device memory) through the C ABI: two calls in a row, the
second on a smaller batch, each bit-identical to rk_masked_attn_fwd with a
caller workspace on the same inputs (same kernels, same order of work).
The first call keeps its rotated keys and the partial results of split key
ranges in the library's scratch array, the second only its rotated keys.
"""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

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


def _case(rk, wl, candidates_only):
    batch = rk.Batch.from_workload(wl)
    plan = rk.Plan(batch, delay=wl.delay, window=wl.window, num_heads=wl.heads,
                   candidates_only=candidates_only)
    q, k, v = (torch.from_numpy(x).cuda().to(torch.bfloat16) for x in (wl.q, wl.k, wl.v))
    return batch, plan, q, k, v


@pytest.mark.parametrize("first", ["serving-split", "plain"])
def test_noalloc_matches_workspace_call(rk, first):
    rng = np.random.default_rng(77)
    # a serving call: few candidate tiles, so their key ranges are split
    # across workgroups (partial results in the scratch array), K rotated by
    # the call (rotated keys in the scratch array)
    serving = make_custom([[(HISTORY, np.sort(rng.integers(NOW - 10**7, NOW - 60, 3000))),
                            (CANDIDATE, np.full(64, NOW, np.int64))] for _ in range(4)],
                          heads=2, d_head=64, dtype="bf16", seed=77, window=500,
                          name="serving-split")
    plain = make_custom([[(HISTORY, np.sort(rng.integers(NOW - 10**6, NOW, 500)))],
                         [(HISTORY, np.sort(rng.integers(NOW - 10**6, NOW - 60, 300))),
                          (CANDIDATE, np.full(9, NOW, np.int64))]],
                        heads=2, d_head=64, dtype="bf16", seed=78, delay=3600, name="plain")
    order = [(serving, True), (plain, False)] if first == "serving-split" else [
        (plain, False), (serving, True)]
    for wl, cand in order:
        _say(f"[gpu] no-alloc forward {wl.name}: T={wl.total_tokens}")
        batch, plan, q, k, v = _case(rk, wl, cand)
        if cand:
            st = plan.stats()
            assert st["split_items"] > 0
        o_ref = torch.zeros_like(q)
        l_ref = torch.zeros((wl.heads, wl.total_tokens), dtype=torch.float32, device="cuda")
        rk.rk_masked_attn_fwd(plan, q, k, v, out=o_ref, lse=l_ref, rope=_rope(wl))
        o = torch.zeros_like(q)
        lse = torch.zeros_like(l_ref)
        rk.rk_masked_attn_fwd_noalloc(plan, q, k, v, out=o, lse=lse, rope=_rope(wl))
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref)
        assert torch.equal(lse, l_ref)
        plan.close()


def test_noalloc_rejects_workspace_and_oversize(rk):
    """A passed workspace is an invalid argument; a call whose rotated keys
    exceed the scratch array is refused before any work (zero-stride views
    stand in for 1.1 M tokens x 2 heads of bf16 keys, 281 MB)."""
    import ctypes as C

    from masked_attention_amd import _rk
    T = 1_100_000
    R = T // 250
    reqs = [[(HISTORY, np.arange(NOW - 250, NOW, dtype=np.int64))] for _ in range(R)]
    wl = make_custom(reqs, heads=2, d_head=64, dtype="bf16", with_qkv=False, name="big")
    batch = rk.Batch.from_workload(wl)
    plan = rk.Plan(batch, num_heads=2)
    x = torch.zeros((1, 2, 64), dtype=torch.bfloat16, device="cuda").expand(T, 2, 64)
    o = torch.zeros((1, 2, 64), dtype=torch.bfloat16, device="cuda").expand(T, 2, 64)
    rp = rk.binding.rope_params(**_rope(wl))
    a = rk.binding._attn_args(plan, x, x, x, o, None, 0.0, rp, False, None)
    st = _rk.lib().rk_masked_attn_fwd_noalloc(plan.handle, C.byref(a), None)
    assert st == _rk.RK_ERR_WORKSPACE_TOO_SMALL
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    a.workspace = ws.data_ptr()
    a.workspace_bytes = 256
    st = _rk.lib().rk_masked_attn_fwd_noalloc(plan.handle, C.byref(a), None)
    assert st == _rk.RK_ERR_INVALID_ARG
    torch.cuda.synchronize()
    plan.close()
