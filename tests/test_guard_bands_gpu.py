"""Guard bands: every buffer the library writes (plan workspace, attention
workspace, rotated K, O, LSE) sits between two 4 KiB canary margins filled
with 0xA5; after the planner, the rotation and the attention have run (and
the plan totals were read), both margins of every buffer must be unchanged.
Covers the MFMA kernel (bf16, d = 64, fused and pre-rotated K), the plain
kernel (fp32, d = 32 and 128), ragged layouts with every mask mode, and
split serving calls, whose attention workspace also holds partial results."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from rk_workloads import (CANDIDATE, HISTORY, make_config, make_custom,  # noqa: E402
                          random_layout)

pytestmark = pytest.mark.gpu

G = 4096          # canary bytes on each side (a multiple of 256 keeps alignment)
CANARY = 0xA5


@pytest.fixture(scope="module")
def rk():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import masked_attention_amd as m
    from masked_attention_amd import _rk
    _rk.lib()
    return m


class Guarded:
    """A device byte buffer with canary margins; `inner` is what the library sees."""

    def __init__(self, nbytes: int):
        self.n = int(nbytes)
        self.buf = torch.full((G + self.n + G,), CANARY, dtype=torch.uint8, device="cuda")
        self.inner = self.buf[G:G + self.n]

    def typed(self, dtype, shape):
        return self.inner.view(dtype).view(*shape)

    def intact(self) -> bool:
        lo = self.buf[:G]
        hi = self.buf[G + self.n:]
        return bool(torch.all(lo == CANARY).item()) and bool(torch.all(hi == CANARY).item())


def _run_guarded(rk, wl, *, rope=True, prerotate=False, reference=False, candidates_only=False):
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    esz = 2 if wl.dtype == "bf16" else 4
    T, H, d = wl.total_tokens, wl.heads, wl.d_head
    batch = rk.Batch.from_workload(wl)
    guards = []

    wsp = Guarded(rk.rk_plan_workspace_size(batch, H))
    guards.append(("plan workspace", wsp))
    plan = rk.Plan(batch, delay=wl.delay, window=wl.window,
                   static_bidirectional=wl.static_bidirectional, num_heads=H,
                   workspace=wsp.inner, candidates_only=candidates_only)
    q, k, v = (torch.from_numpy(x).to("cuda").to(dt) for x in (wl.q, wl.k, wl.v))
    rp = dict(phi_min=wl.phi_min, dt_max=wl.dt_max, base=wl.base) if rope else None
    if prerotate:
        kr = Guarded(T * H * d * esz)
        guards.append(("rotated K", kr))
        k = rk.rk_time_rope(batch, k, out=kr.typed(dt, (T, H, d)), **rp)
    og = Guarded(T * H * d * esz)
    lg = Guarded(H * T * 4)
    guards += [("O", og), ("LSE", lg)]
    n = rk.rk_attn_workspace_size(plan, q, k, v, rope=rp, reference=reference,
                                  k_prerotated=prerotate)
    wa = None
    if n:
        wa = Guarded(n)
        guards.append(("attention workspace", wa))
    o, lse = rk.rk_masked_attn_fwd(plan, q, k, v, out=og.typed(dt, (T, H, d)),
                                   lse=lg.typed(torch.float32, (H, T)), rope=rp,
                                   reference=reference, k_prerotated=prerotate,
                                   workspace=wa.inner if wa is not None else None)
    st = plan.stats()
    torch.cuda.synchronize()
    assert st["device_errors"] == 0
    if candidates_only:
        assert st["split_items"] > 0, "layout meant to split produced no split item"
    else:
        assert torch.isfinite(o.float()).all()
    for name, g in guards:
        assert g.intact(), f"{wl.name}: canary of {name} overwritten"
    plan.close()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_guard_bands_random_layouts(rk, seed):
    rng = np.random.default_rng(300 + seed)
    reqs = random_layout(rng, 6, 700)
    for dtype, d in (("bf16", 64), ("f32", 32), ("f32", 128)):
        for bidir, delay, window in ((False, 0, 0), (False, 3600, 0), (False, 0, 100),
                                     (True, 0, 0)):
            wl = make_custom(reqs, heads=2, d_head=d, dtype=dtype, delay=delay, window=window,
                             static_bidirectional=bidir, seed=seed,
                             name=f"guard-{seed}-{dtype}-{d}")
            _run_guarded(rk, wl)


def test_guard_bands_prerotated_and_reference(rk):
    wl = make_custom(random_layout(np.random.default_rng(310), 4, 900), heads=2, d_head=64,
                     dtype="bf16", seed=310, delay=600, name="guard-prerot")
    _run_guarded(rk, wl, prerotate=True)
    _run_guarded(rk, wl, reference=True)
    _run_guarded(rk, wl, rope=False)


@pytest.mark.parametrize("cfg", [3, 4])
def test_guard_bands_workloads(rk, cfg):
    _run_guarded(rk, make_config(cfg))


@pytest.mark.parametrize("dtype,d,reference", [("bf16", 64, False), ("bf16", 64, True),
                                               ("f32", 128, False)])
def test_guard_bands_split(rk, dtype, d, reference):
    rng = np.random.default_rng(320)
    reqs = random_layout(rng, 3, 3000, kinds=(HISTORY, CANDIDATE), allow_empty=False)
    wl = make_custom(reqs, heads=2, d_head=d, dtype=dtype, seed=320, name="guard-split")
    _run_guarded(rk, wl, reference=reference, candidates_only=True)
    _run_guarded(rk, wl, rope=False, reference=reference, candidates_only=True)
