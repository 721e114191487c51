"""GPU parity of the LazFormer pre-passes (section 2.3) through the C ABI.

* rk_gather_mean with the pooled layouts of rk_prune_layout_ex (SORT query
  pruning, exponential and linear schedules) against the oracle;
* rk_gather_sum applied with the layouts of rk_compress_layout /
  rk_prune_layout reproduces the oracle's compressed / pruned rows: fp32
  within 1e-5 relative to the row magnitude, bf16 within one bf16 rounding
  (2^-8 relative) of the oracle's fp64 sums; vectorised and scalar paths,
  padded row strides; ranges outside the input are clamped.
* End to end: compress Q, K, V on the device, plan the compressed batch
  with the LazFormer mask (window W, global tail G, targets see the
  history and themselves), run the attention, then prune to each layer's
  input and run it again; every layer's output equals the oracle attention
  on the oracle's compressed and pruned inputs (bf16: relative L2 within
  1e-2; max-abs within 2e-2 * max(1, max |reference|), since group sums of
  unit-variance rows give outputs near 10 in magnitude and sharper scores).
"""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from rk_workloads import (CANDIDATE, HISTORY, NOW, bf16_round, history_span,  # noqa: E402
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


def _close(got, ref, dtype):
    scale = np.maximum(np.abs(ref), 1.0)
    tol = 1e-5 if dtype == torch.float32 else 2.0 ** -8
    assert np.all(np.abs(got - ref) <= tol * scale), np.abs(got - ref).max()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
# widths that pack 8, 4, 2 and 1 output rows per wave (16-byte lanes: 64 bf16 = 8 lanes,
# 128 = 16, 256 = 32, 512 = 64) and unaligned widths on the element-per-lane form (13: four
# rows per wave, 37: one)
@pytest.mark.parametrize("width,pad", [(64, 0), (128, 8), (256, 0), (512, 8), (13, 3),
                                       (37, 3)])
def test_gather_sum_compress_and_prune(rk, dtype, width, pad):
    rng = np.random.default_rng(width + pad)
    wl = make_custom(random_layout(rng, 9, 600), heads=1, d_head=2, seed=1, with_qkv=False)
    x = rng.standard_normal((wl.total_tokens, width)).astype(np.float32)
    if dtype == torch.bfloat16:
        x = bf16_round(x)
    big = torch.zeros((wl.total_tokens, width + pad), dtype=dtype, device="cuda")
    big[:, :width] = torch.from_numpy(x).to(dtype)
    xd = big[:, :width]
    lay = rk.Layout.from_workload(wl)
    for keep, group in ((16, 8), (0, 3), (100, 1)):
        _say(f"[gpu] gather_sum compress {dtype} width={width} pad={pad} keep={keep} g={group}")
        out = rk.rk_compress_layout(lay, keep=keep, group=group)
        rg = torch.from_numpy(out.ranges.copy()).cuda()
        yb = torch.full((out.T, width + pad), 7.0, dtype=dtype, device="cuda")
        rk.rk_gather_sum(rg, xd, out=yb[:, :width])
        torch.cuda.synchronize()
        _, _, _, ref = oracle.group_sum_compress(wl.req_offsets, wl.seg_kind, wl.timestamps,
                                                 x.astype(np.float64), keep=keep, group=group)
        _close(yb[:, :width].float().cpu().numpy(), ref, dtype)
        assert torch.all(yb[:, width:] == 7.0)  # padding untouched
    lt = lay.history_lengths()
    for layer in (2, 4):
        _say(f"[gpu] gather_sum prune {dtype} width={width} layer={layer}")
        out = rk.rk_prune_layout(lay, l_tilde=lt, n_min=32, layer=layer, num_layers=4)
        y = rk.rk_gather_sum(torch.from_numpy(out.ranges.copy()).cuda(), xd)
        torch.cuda.synchronize()
        _, _, _, ref = oracle.prune_history(wl.req_offsets, wl.seg_kind, wl.timestamps, x,
                                            l_tilde=lt, n_min=32, layer=layer, num_layers=4)
        assert np.array_equal(y.float().cpu().numpy(), ref.astype(np.float32))


def test_gather_sum_clamps_ranges(rk):
    x = torch.arange(20, dtype=torch.float32, device="cuda").reshape(10, 2)
    rg = torch.tensor([[-5, 2], [8, 50], [7, 3], [3, 4]], dtype=torch.int32, device="cuda")
    y = rk.rk_gather_sum(rg, x)
    torch.cuda.synchronize()
    assert y.cpu().tolist() == [[2.0, 4.0], [34.0, 36.0], [0.0, 0.0], [6.0, 7.0]]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("width,pad", [(64, 0), (256, 0), (13, 3), (37, 3)])
def test_gather_mean_pooled_pruning(rk, dtype, width, pad):
    """SORT's pooled query pruning (section 3.2.2): rk_prune_layout_ex's
    ranges moved by rk_gather_mean against the oracle's pooled layer input,
    exponential and linear schedules; padding columns untouched."""
    rng = np.random.default_rng(900 + width)
    wl = make_custom(random_layout(rng, 9, 600), heads=1, d_head=2, seed=2, with_qkv=False)
    x = rng.standard_normal((wl.total_tokens, width)).astype(np.float32)
    if dtype == torch.bfloat16:
        x = bf16_round(x)
    big = torch.zeros((wl.total_tokens, width + pad), dtype=dtype, device="cuda")
    big[:, :width] = torch.from_numpy(x).to(dtype)
    xd = big[:, :width]
    lay = rk.Layout.from_workload(wl)
    lt = lay.history_lengths()
    for schedule, layer in (("exp", 2), ("exp", 4), ("linear", 3)):
        _say(f"[gpu] gather_mean pooled {dtype} width={width} pad={pad} {schedule} layer={layer}")
        out = rk.rk_prune_layout_ex(lay, l_tilde=lt, schedule=schedule, n_min=16, layer=layer,
                                    num_layers=4, decay=0.5, pool=True)
        if schedule == "exp":
            keep = [oracle.pruned_history_length_exp(int(l), 16, 0.5, layer) for l in lt]
        else:
            keep = [oracle.pruned_history_length(int(l), 16, layer, 4) for l in lt]
        rg = torch.from_numpy(out.ranges.copy()).cuda()
        yb = torch.full((out.T, width + pad), 7.0, dtype=dtype, device="cuda")
        rk.rk_gather_mean(rg, xd, out=yb[:, :width])
        torch.cuda.synchronize()
        _, _, _, ref = oracle.prune_history_pooled(wl.req_offsets, wl.seg_kind, wl.timestamps,
                                                   x.astype(np.float64), keep=keep)
        _close(yb[:, :width].float().cpu().numpy(), ref, dtype)
        assert torch.all(yb[:, width:] == 7.0)


def test_gather_mean_clamps_ranges(rk):
    x = torch.arange(20, dtype=torch.float32, device="cuda").reshape(10, 2)
    rg = torch.tensor([[-5, 2], [8, 50], [7, 3], [3, 4]], dtype=torch.int32, device="cuda")
    y = rk.rk_gather_mean(rg, x)
    torch.cuda.synchronize()
    # clamped to [0, 2), [8, 10), empty, [3, 4)
    assert y.cpu().tolist() == [[1.0, 2.0], [17.0, 18.0], [0.0, 0.0], [6.0, 7.0]]


def _lazformer_batch(R, L_hist, n_cand, H, d, seed):
    rng = np.random.default_rng(seed)
    reqs = []
    for r in range(R):
        Lh = L_hist - 37 * r  # ragged histories
        reqs.append([(HISTORY, history_span(rng, Lh, NOW - 60)),
                     (CANDIDATE, np.full(n_cand, NOW, np.int64))])
    return make_custom(reqs, heads=H, d_head=d, dtype="bf16", seed=seed)


def test_lazformer_stack_end_to_end(rk):
    """Compression 2048 -> 1024 + 128 groups of 8 is scaled down here to
    history 700 (keep 300, groups of 8), W = G = N_min = 64, 4 layers."""
    H, d = 2, 64
    wl = _lazformer_batch(3, 700, 40, H, d, seed=5)
    keep, group, W, G, n_min, n_layers = 300, 8, 64, 64, 64, 4
    rope = dict(phi_min=wl.phi_min, dt_max=wl.dt_max, base=wl.base)
    lay = rk.Layout.from_workload(wl)
    comp = rk.rk_compress_layout(lay, keep=keep, group=group)
    rg = torch.from_numpy(comp.ranges.copy()).cuda()
    qkv = [torch.from_numpy(a).cuda().to(torch.bfloat16) for a in (wl.q, wl.k, wl.v)]
    cq, ck, cv = (rk.rk_gather_sum(rg, t) for t in qkv)
    # oracle compression of the same bf16 inputs
    ref_c = [oracle.group_sum_compress(wl.req_offsets, wl.seg_kind, wl.timestamps,
                                       a.astype(np.float64), keep=keep, group=group)
             for a in (wl.q, wl.k, wl.v)]
    offs, kinds, times = ref_c[0][0], ref_c[0][1], ref_c[0][2]
    assert np.array_equal(offs, comp.req_offsets) and np.array_equal(kinds, comp.seg_kind)
    # the device sums are rounded to bf16; the oracle attention takes those rounded values
    torch.cuda.synchronize()
    comp_np = [t.float().cpu().numpy() for t in (cq, ck, cv)]
    for a, rc in zip(comp_np, ref_c):
        _close(a, rc[3], torch.bfloat16)
    lt = comp.history_lengths()
    cur_lay, cur = comp, (cq, ck, cv)
    cur_np = comp_np
    for layer in range(1, n_layers + 1):
        _say(f"[gpu] lazformer layer {layer}")
        lay_l = rk.rk_prune_layout(comp, l_tilde=lt, n_min=n_min, layer=layer,
                                   num_layers=n_layers)
        rgl = torch.from_numpy(lay_l.ranges.copy()).cuda()
        ql, kl, vl = (rk.rk_gather_sum(rgl, t) for t in (cq, ck, cv))
        anchors = np.full(lay_l.R, NOW, np.int64)
        batch = rk.Batch(lay_l.req_offsets, lay_l.seg_kind, lay_l.timestamps, anchors)
        plan = rk.Plan(batch, window=W, global_tail=G, num_heads=H)
        o, _ = rk.rk_masked_attn_fwd(plan, ql, kl, vl, rope=rope)
        torch.cuda.synchronize()
        sel = np.concatenate([np.arange(b, e) for b, e in lay_l.ranges]) if lay_l.T else []
        qn, kn, vn = (a[sel] for a in comp_np)
        ref, _ = oracle.attention_forward(lay_l.req_offsets, lay_l.seg_kind, lay_l.timestamps,
                                          qn.astype(np.float64), kn.astype(np.float64),
                                          vn.astype(np.float64), delay=0, window=W,
                                          static_bidirectional=False, rope=rope, global_tail=G)
        got = o.float().cpu().numpy().astype(np.float64)
        err = np.abs(got - ref).max()
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        # group sums of N(0,1) rows reach |O| ~ 10: max-abs is bounded relative
        # to the output's magnitude, relative L2 by 1e-2 as for unit inputs
        bound = 2e-2 * max(1.0, float(np.abs(ref).max()))
        assert err <= bound and rel <= 1e-2, (layer, err, bound, rel)
        n_hist = [rk.rk_pruned_history_length(int(x), n_min, layer, n_layers) for x in lt]
        assert lay_l.history_lengths().tolist() == [min(a, b) for a, b in zip(n_hist, lt)]
        plan.close()
