"""CPU fp64 oracle for request-centric masked attention with time RoPE.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module; only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP library: it
builds the explicit visibility matrix of every request pair by pair and runs
plain softmax attention in float64, and takes the gradients of that
definition by the chain rule for the backward.

Sources (pages as they appear in the reference text):

* CADET (paper-daily.com "CADET: Context-Conditioned Ads CTR Prediction With
  a Decoder-Only Transformer"):
  - section "why mask the most recent hour in training", equation
    M_ij = -inf if t_j > t_i - Delta_delay            -> delay rule
  - section "time encoding and self-gating", equation
    alpha_i(t) = t * phi_min / Delta_t_max * base^(2i/d) -> time RoPE
  - section "how to score hundreds of candidates in 50 ms": candidates are
    appended after the user sequence and see the history but not each other.
* SORT (10100.com article 149105610), section 3.1: U2U sees only its past,
  C2U sees all user features, C2C isolated; section 3.2.1: sliding window in
  U2U only.
* LazFormer (liuzhao09.github.io lazformer page), section 2.3 equations 19-21:
  allowed relation A(p, q) with window W, targets-to-history and target
  self-links; masked entries are -inf and SparseAttn = softmax(QK^T/sqrt(d_k)
  + M) V.
* MTGR (joezjh.github.io blog index, "MTGR", model-structure part): static
  profile + history mutually visible, real-time sequence causal, each target
  sees the static tokens plus the real-time events before its own time, and
  no other target.
* TM20K (liuzhao09.github.io tm20k page, section 2.1 equations): scaled
  dot-product attention with an additive mask.

Readings taken where the pages are silent or ambiguous (each one is listed in
the design notes of the repository as well):

* pair index i of the rotation runs 0 .. d/2-1 and pairs adjacent components
  (2i, 2i+1); the rotation is counter-clockwise;
* the softmax scale is 1/sqrt(d_head);
* the delay rule is literal (hidden iff t_j > t_i - Delta), so with Delta > 0
  a token does not see itself; Delta = 0 switches the time condition off;
* the delay and the window apply to static-to-static (U2U) pairs only; the
  window keeps keys with p_i - p_j < W;
* real-time to real-time is p_j <= p_i and t_j <= t_i; target to real-time is
  t_j < t_i ("before");
* a row with no visible key outputs 0 and has log-sum-exp -inf.
* SORT section 3.2.2 (query pruning) names linear, exponential and pooling
  strategies whose formulas did not survive on the page: the exponential
  schedule is read as N^l = min(L~, max(N_min, Round(L~ * decay^(l - 1))))
  and pooling as the pruned history tokens of a request averaged into one
  token placed where they were and dated as their newest member.  The pins
  of these two check the oracle against that reading (closed forms,
  conservation of the history total, brute force); the reading itself has
  no printed formula to be pinned to.
"""

from __future__ import annotations

import math
from typing import Dict, Optional, Tuple

import numpy as np

PROFILE, HISTORY, REALTIME, CANDIDATE = 0, 1, 2, 3
EMPTY, PARTIAL, FULL = 0, 1, 2
TILE_Q, TILE_K = 128, 64


# ---------------------------------------------------------------------------
# Visibility rule (explicit, per pair)
# ---------------------------------------------------------------------------

def visible_rows(seg_kind: np.ndarray, timestamps: np.ndarray, rows: np.ndarray, *,
                 delay: int, window: int, static_bidirectional: bool,
                 global_tail: int = 0, cols: Optional[np.ndarray] = None) -> np.ndarray:
    """Visibility of every key (or of the keys `cols`) for the query rows
    `rows` of ONE request.

    Returns a bool array [len(rows), L] (or [len(rows), len(cols)]): True
    where query i may attend key j.  Each entry is the rule applied to the
    pair (i, j) on its own; evaluating a subset of rows or keys gives the same
    entries as the full matrix.

    global_tail (LazFormer section 2.3, eq. 19-21, G): the last G static
    (profile + history) positions are global queries, exempt from the
    window; they still see only earlier keys, and the delay still applies.
    """
    seg_kind = np.asarray(seg_kind)
    t = np.asarray(timestamps, dtype=np.int64)
    L = seg_kind.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.arange(L, dtype=np.int64) if cols is None else np.asarray(cols, dtype=np.int64)
    pi = rows[:, None]
    pj = cols[None, :]
    si = seg_kind[rows][:, None]
    sj = seg_kind[cols][None, :]
    ti = t[rows][:, None]
    tj = t[cols][None, :]

    static_i = (si == PROFILE) | (si == HISTORY)
    static_j = (sj == PROFILE) | (sj == HISTORY)
    n_static = int(np.count_nonzero((seg_kind == PROFILE) | (seg_kind == HISTORY)))

    # key is a candidate: only the diagonal (C2C isolation, and U2C never)
    vis = (sj == CANDIDATE) & (pi == pj)

    # static query -> static key (U2U)
    if static_bidirectional:
        u2u = np.ones_like(vis)
    else:
        u2u = pj <= pi
        if window > 0:
            u2u = u2u & ((pi - pj < window) | (pi >= n_static - global_tail))
        if delay > 0:
            u2u = u2u & ~(tj > ti - delay)
    vis |= static_i & static_j & u2u

    # real-time query: sees every static key, and real-time keys up to itself
    rt_i = si == REALTIME
    vis |= rt_i & static_j
    vis |= rt_i & (sj == REALTIME) & (pj <= pi) & (tj <= ti)

    # candidate query: every static key (C2U) and real-time keys strictly before it
    c_i = si == CANDIDATE
    vis |= c_i & static_j
    vis |= c_i & (sj == REALTIME) & (tj < ti)
    return vis


def visibility(seg_kind: np.ndarray, timestamps: np.ndarray, *, delay: int, window: int,
               static_bidirectional: bool, global_tail: int = 0) -> np.ndarray:
    """Full L x L visibility matrix of one request."""
    L = np.asarray(seg_kind).shape[0]
    return visible_rows(seg_kind, timestamps, np.arange(L), delay=delay, window=window,
                        static_bidirectional=static_bidirectional, global_tail=global_tail)


def count_visible(seg_kind, timestamps, *, delay, window, static_bidirectional,
                  global_tail: int = 0, row_block: int = 1024) -> int:
    """Number of visible (query, key) pairs of one request."""
    L = np.asarray(seg_kind).shape[0]
    total = 0
    for r0 in range(0, L, row_block):
        rows = np.arange(r0, min(L, r0 + row_block))
        total += int(np.count_nonzero(visible_rows(seg_kind, timestamps, rows, delay=delay,
                                                   window=window,
                                                   static_bidirectional=static_bidirectional,
                                                   global_tail=global_tail)))
    return total


# ---------------------------------------------------------------------------
# Time RoPE (CADET, time-encoding section)
# ---------------------------------------------------------------------------

def rope_frequencies(d: int, phi_min: float, dt_max: float, base: float) -> np.ndarray:
    """omega_i = phi_min / dt_max * base^(2i/d), i = 0 .. d/2-1 (radians per time unit)."""
    i = np.arange(d // 2, dtype=np.float64)
    return phi_min / dt_max * np.power(float(base), 2.0 * i / d)


def time_rope(x: np.ndarray, t: np.ndarray, *, phi_min: float, dt_max: float,
              base: float) -> np.ndarray:
    """Rotate pairs (2i, 2i+1) of x[..., d] by alpha_i(t) = t * omega_i.

    x has shape [N, ..., d]; t has shape [N] (one time per token, shared by
    every head).  Computed in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    omega = rope_frequencies(d, phi_min, dt_max, base)
    t = np.asarray(t, dtype=np.float64).reshape((-1,) + (1,) * (x.ndim - 1))
    alpha = t * omega                      # [N, 1.., d/2]
    c, s = np.cos(alpha), np.sin(alpha)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


def qk_rmsnorm(x: np.ndarray, gamma: Optional[np.ndarray], eps: float) -> np.ndarray:
    """QK Norm (TM20K section 2; SORT section 3.3.2: RMSNorm on Q and K before
    the scores): every [d] row x becomes x / sqrt(mean(x^2) + eps) * gamma
    (gamma None = 1).  float64."""
    x = np.asarray(x, np.float64)
    y = x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    return y if gamma is None else y * np.asarray(gamma, np.float64)


# ---------------------------------------------------------------------------
# Masked softmax attention (plain definition)
# ---------------------------------------------------------------------------

def masked_softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, vis: np.ndarray,
                             scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """softmax(q k^T * scale + M) v for one head, M = 0 where vis else -inf.

    q [Lq, d], k [Lk, d], v [Lk, d], vis bool [Lq, Lk].  Returns (o [Lq, d],
    lse [Lq]) where lse is the natural log of the softmax denominator of the
    scaled scores.  A row with no visible key gives o = 0 and lse = -inf.
    """
    s = (q @ k.T) * scale
    s = np.where(vis, s, -np.inf)
    has = vis.any(axis=1)
    m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.exp(s - m[:, None])             # exp(-inf) = 0 on hidden keys
    denom = e.sum(axis=1)
    o = np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    o[has] = (e[has] @ v) / denom[has, None]
    lse = np.full(q.shape[0], -np.inf)
    lse[has] = m[has] + np.log(denom[has])
    return o, lse


def attention_forward(req_offsets: np.ndarray, seg_kind: np.ndarray, timestamps: np.ndarray,
                      q: np.ndarray, k: np.ndarray, v: np.ndarray, *, delay: int, window: int,
                      static_bidirectional: bool, rope: Optional[Dict[str, float]] = None,
                      rope_times: Optional[np.ndarray] = None, scale: Optional[float] = None,
                      heads: Optional[np.ndarray] = None, requests: Optional[np.ndarray] = None,
                      row_block: int = 1024, global_tail: int = 0,
                      qk_norm: Optional[Dict] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Masked attention forward over a packed batch, in float64.

    qk_norm: None or dict(eps=..., gamma_q=..., gamma_k=...): QK Norm of q and
    k (qk_rmsnorm) before the rotation.

    q, k, v: [T, H, d] (any float dtype; upcast to float64).  With `rope`
    (keys phi_min, dt_max, base) Q and K are rotated by time RoPE using
    `rope_times` (default: the absolute timestamps).  Returns o [T, H, d] and
    lse [H, T].  `heads` / `requests` restrict the work to a subset (other
    entries stay 0 / -inf).  Rows are processed in blocks of `row_block`;
    every row's softmax is independent, so blocking does not change results.
    """
    T, H, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    if qk_norm is not None:
        q = qk_rmsnorm(q, qk_norm.get("gamma_q"), qk_norm["eps"])
        k = qk_rmsnorm(k, qk_norm.get("gamma_k"), qk_norm["eps"])
    o = np.zeros((T, H, d), np.float64)
    lse = np.full((H, T), -np.inf)
    heads = np.arange(H) if heads is None else np.asarray(heads)
    R = req_offsets.shape[0] - 1
    requests = np.arange(R) if requests is None else np.asarray(requests)
    if rope is not None:
        tr = timestamps if rope_times is None else rope_times
    for r in requests:
        a, b = int(req_offsets[r]), int(req_offsets[r + 1])
        L = b - a
        if L == 0:
            continue
        sk, ts = seg_kind[a:b], timestamps[a:b]
        qr, kr, vr = q[a:b], k[a:b], v[a:b]
        if rope is not None:
            qr = time_rope(qr, tr[a:b], **rope)
            kr = time_rope(kr, tr[a:b], **rope)
        for r0 in range(0, L, row_block):
            rows = np.arange(r0, min(L, r0 + row_block))
            vis = visible_rows(sk, ts, rows, delay=delay, window=window,
                               static_bidirectional=static_bidirectional,
                               global_tail=global_tail)
            for h in heads:
                oh, lh = masked_softmax_attention(qr[rows, h], kr[:, h], vr[:, h], vis, scale)
                o[a + rows, h] = oh
                lse[h, a + rows] = lh
    return o, lse


def attention_rows(req_offsets, seg_kind, timestamps, q, k, v, tokens: np.ndarray,
                   head: int, *, delay, window, static_bidirectional, rope=None,
                   rope_times=None, scale=None, global_tail: int = 0):
    """Output rows for selected global tokens of one head (for sampled checks).

    Each token is computed against its own request's keys, exactly as in
    attention_forward.  Returns (o [n, d], lse [n]).
    """
    T, H, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    tokens = np.asarray(tokens, np.int64)
    req_of = np.searchsorted(req_offsets, tokens, side="right") - 1
    o = np.zeros((tokens.shape[0], d))
    lse = np.full(tokens.shape[0], -np.inf)
    tr = timestamps if rope_times is None else rope_times
    for r in np.unique(req_of):
        sel = np.nonzero(req_of == r)[0]
        a, b = int(req_offsets[r]), int(req_offsets[r + 1])
        rows = tokens[sel] - a
        sk, ts = seg_kind[a:b], timestamps[a:b]
        qr = np.asarray(q[a + rows, head], np.float64)
        kr = np.asarray(k[a:b, head], np.float64)
        vr = np.asarray(v[a:b, head], np.float64)
        if rope is not None:
            qr = time_rope(qr, tr[a + rows], **rope)
            kr = time_rope(kr, tr[a:b], **rope)
        vis = visible_rows(sk, ts, rows, delay=delay, window=window,
                           static_bidirectional=static_bidirectional, global_tail=global_tail)
        oh, lh = masked_softmax_attention(qr, kr, vr, vis, scale)
        o[sel] = oh
        lse[sel] = lh
    return o, lse


# ---------------------------------------------------------------------------
# HSTU pointwise aggregated attention (HSTU, eq. 2)
# ---------------------------------------------------------------------------

def time_bucket(dt: int, num_buckets: int) -> int:
    """Bucket of a time difference: floor(log2(1 + |dt|)) capped at
    num_buckets - 1 (exact integer arithmetic: the bit length of 1 + |dt|
    minus one)."""
    return min(int(1 + abs(int(dt))).bit_length() - 1, num_buckets - 1)


def hstu_rab(positions: np.ndarray, times: np.ndarray, rows: np.ndarray,
             pos_bias: Optional[np.ndarray], time_bias: Optional[np.ndarray]) -> np.ndarray:
    """Relative attention bias rab^{p,t} [len(rows), L] of one request, shared
    by every head: pos_bias[min(|p_i - p_j|, P - 1)] + time_bias[bucket of
    t_i - t_j] (time_bucket).  A None table contributes 0."""
    rows = np.asarray(rows, np.int64)
    L = positions.shape[0]
    rab = np.zeros((rows.shape[0], L))
    if pos_bias is not None:
        dp = np.abs(positions[rows][:, None] - positions[None, :])
        rab += np.asarray(pos_bias, np.float64)[np.minimum(dp, len(pos_bias) - 1)]
    if time_bias is not None:
        B = len(time_bias)
        dt = np.abs(np.asarray(times, np.int64)[rows][:, None] - np.asarray(times, np.int64)[None, :])
        # bit length of 1 + |dt| minus one, capped
        bucket = np.minimum(np.floor(np.log2(1.0 + dt.astype(np.float64))).astype(np.int64), B - 1)
        # float log2 can round up just below a power of two: correct by integers
        bucket = np.where((np.left_shift(np.int64(1), np.maximum(bucket, 0)) > 1 + dt), bucket - 1,
                          bucket)
        rab += np.asarray(time_bias, np.float64)[np.clip(bucket, 0, B - 1)]
    return rab


def pointwise_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, vis: np.ndarray,
                        scale: float, rab: Optional[np.ndarray]) -> np.ndarray:
    """HSTU eq. 2 for one head: O = (SiLU(q k^T * scale + rab) * vis) v, with
    SiLU(x) = x / (1 + exp(-x)); masked pairs contribute nothing and there is
    no normalisation."""
    x = (q @ k.T) * scale
    if rab is not None:
        x = x + rab
    w = np.where(vis, x / (1.0 + np.exp(-x)), 0.0)
    return w @ v


def pointwise_attention_forward(req_offsets, seg_kind, timestamps, q, k, v, *, delay, window,
                                static_bidirectional, scale: float = 1.0, pos_bias=None,
                                time_bias=None, global_tail: int = 0, heads=None,
                                requests=None, row_block: int = 1024) -> np.ndarray:
    """HSTU pointwise attention over a packed batch with the method's mask
    (each request's explicit visibility), float64.  Returns o [T, H, d]."""
    T, H, d = q.shape
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    o = np.zeros((T, H, d))
    heads = np.arange(H) if heads is None else np.asarray(heads)
    R = req_offsets.shape[0] - 1
    requests = np.arange(R) if requests is None else np.asarray(requests)
    for r in requests:
        a, b = int(req_offsets[r]), int(req_offsets[r + 1])
        L = b - a
        if L == 0:
            continue
        pos = np.arange(L, dtype=np.int64)
        for r0 in range(0, L, row_block):
            rows = np.arange(r0, min(L, r0 + row_block))
            vis = visible_rows(seg_kind[a:b], timestamps[a:b], rows, delay=delay, window=window,
                               static_bidirectional=static_bidirectional,
                               global_tail=global_tail)
            rab = hstu_rab(pos, timestamps[a:b], rows, pos_bias, time_bias)
            for h in heads:
                o[a + rows, h] = pointwise_attention(q[a + rows, h], k[a:b, h], v[a:b, h], vis,
                                                     scale, rab)
    return o


def pointwise_attention_rows(req_offsets, seg_kind, timestamps, q, k, v, tokens, head, *, delay,
                             window, static_bidirectional, scale: float = 1.0, pos_bias=None,
                             time_bias=None, global_tail: int = 0) -> np.ndarray:
    """Pointwise attention output rows of selected global tokens of one head
    (for sampled checks); each token against its own request's keys."""
    tokens = np.asarray(tokens, np.int64)
    d = q.shape[-1]
    req_of = np.searchsorted(req_offsets, tokens, side="right") - 1
    o = np.zeros((tokens.shape[0], d))
    for r in np.unique(req_of):
        sel = np.nonzero(req_of == r)[0]
        a, b = int(req_offsets[r]), int(req_offsets[r + 1])
        rows = tokens[sel] - a
        vis = visible_rows(seg_kind[a:b], timestamps[a:b], rows, delay=delay, window=window,
                           static_bidirectional=static_bidirectional, global_tail=global_tail)
        rab = hstu_rab(np.arange(b - a, dtype=np.int64), timestamps[a:b], rows, pos_bias,
                       time_bias)
        o[sel] = pointwise_attention(np.asarray(q[a + rows, head], np.float64),
                                     np.asarray(k[a:b, head], np.float64),
                                     np.asarray(v[a:b, head], np.float64), vis, scale, rab)
    return o


# ---------------------------------------------------------------------------
# Backward of the masked softmax attention (gradients of a scalar loss)
# ---------------------------------------------------------------------------

def masked_softmax_attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                                      do: np.ndarray, vis: np.ndarray, scale: float
                                      ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of a loss with upstream gradient do = dLoss/dO, one head.

    O = P v with P the row softmax of S = q k^T * scale + M (M = 0 where vis,
    -inf elsewhere; a row with no visible key has P = 0 and O = 0).  The
    chain rule through these three steps gives
      dv = P^T do,   dP = do v^T,
      dS_ij = P_ij (dP_ij - sum_l P_il dP_il)      (softmax Jacobian per row),
      dq = scale * dS k,   dk = scale * dS^T q.
    Returns (dq [Lq, d], dk [Lk, d], dv [Lk, d]).
    """
    s = (q @ k.T) * scale
    s = np.where(vis, s, -np.inf)
    has = vis.any(axis=1)
    m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.exp(s - m[:, None])
    denom = np.where(has, e.sum(axis=1), 1.0)
    p = e / denom[:, None]                 # rows without a visible key: all 0
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = (ds @ k) * scale
    dk = (ds.T @ q) * scale
    return dq, dk, dv


def time_rope_transpose(g: np.ndarray, t: np.ndarray, *, phi_min: float, dt_max: float,
                        base: float) -> np.ndarray:
    """Apply the transpose of the time-RoPE rotation to gradients g [N, ..., d].

    Each pair rotation is orthogonal, so its transpose is the rotation by
    -alpha_i(t): the gradient with respect to the unrotated input is
    R(t)^T times the gradient with respect to the rotated one.
    """
    return time_rope(g, -np.asarray(t, dtype=np.float64), phi_min=phi_min, dt_max=dt_max,
                     base=base)


def attention_backward(req_offsets: np.ndarray, seg_kind: np.ndarray, timestamps: np.ndarray,
                       q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, *,
                       delay: int, window: int, static_bidirectional: bool,
                       rope: Optional[Dict[str, float]] = None,
                       rope_times: Optional[np.ndarray] = None, scale: Optional[float] = None,
                       heads: Optional[np.ndarray] = None, requests: Optional[np.ndarray] = None,
                       global_tail: int = 0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients (dq, dk, dv) [T, H, d] of the masked attention forward of
    attention_forward with respect to the unrotated q, k and v, for the
    upstream gradient do [T, H, d], in float64.

    With `rope`, q and k are rotated as in the forward; the gradients with
    respect to the rotated vectors are taken back through the rotation by
    time_rope_transpose.  Every request uses its full explicit L x L mask.
    `heads` / `requests` restrict the work (other entries stay 0).
    """
    T, H, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    dq = np.zeros((T, H, d), np.float64)
    dk = np.zeros((T, H, d), np.float64)
    dv = np.zeros((T, H, d), np.float64)
    heads = np.arange(H) if heads is None else np.asarray(heads)
    R = req_offsets.shape[0] - 1
    requests = np.arange(R) if requests is None else np.asarray(requests)
    if rope is not None:
        tr = timestamps if rope_times is None else rope_times
    for r in requests:
        a, b = int(req_offsets[r]), int(req_offsets[r + 1])
        if b == a:
            continue
        vis = visibility(seg_kind[a:b], timestamps[a:b], delay=delay, window=window,
                         static_bidirectional=static_bidirectional, global_tail=global_tail)
        qr, kr = q[a:b], k[a:b]
        if rope is not None:
            qr = time_rope(qr, tr[a:b], **rope)
            kr = time_rope(kr, tr[a:b], **rope)
        gq = np.zeros((b - a, H, d))
        gk = np.zeros((b - a, H, d))
        for h in heads:
            gq[:, h], gk[:, h], dv[a:b, h] = masked_softmax_attention_backward(
                qr[:, h], kr[:, h], v[a:b, h], do[a:b, h], vis, scale)
        if rope is not None:
            gq = time_rope_transpose(gq, tr[a:b], **rope)
            gk = time_rope_transpose(gk, tr[a:b], **rope)
        dq[a:b, heads] = gq[:, heads]
        dk[a:b, heads] = gk[:, heads]
    return dq, dk, dv


def attention_backward_sampled(req_offsets, seg_kind, timestamps, q, k, v, do, *, request: int,
                               head: int, rows: np.ndarray, keys: np.ndarray, delay, window,
                               static_bidirectional, rope=None, scale=None, global_tail: int = 0,
                               row_block: int = 1024):
    """dq of selected rows and dk, dv of selected keys of ONE request and
    head (request-local positions), for checks at sizes where the full
    matrices do not fit.

    Same chain rule as masked_softmax_attention_backward.  The row softmax
    statistics (log-sum-exp and D_i = do_i . o_i) come first, in blocks of
    rows, for the rows the sampled gradients use: the rows of `rows` and
    every row that sees one of `keys` (any other row has P_ij = 0 for every
    sampled key and enters no sum below); then
      dq_i = scale * sum_j P_ij (dP_ij - D_i) k_j            for i in rows,
      dv_j = sum_i P_ij do_i,
      dk_j = scale * sum_i P_ij (dP_ij - D_i) q_i            for j in keys,
    with the sums over i taken block by block.  Returns (dq [len(rows), d],
    dk [len(keys), d], dv [len(keys), d]) with respect to the unrotated
    vectors.
    """
    a, b = int(req_offsets[request]), int(req_offsets[request + 1])
    L = b - a
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    sk, ts = seg_kind[a:b], timestamps[a:b]
    qr = np.asarray(q[a:b, head], np.float64)
    kr = np.asarray(k[a:b, head], np.float64)
    vr = np.asarray(v[a:b, head], np.float64)
    gr = np.asarray(do[a:b, head], np.float64)
    if rope is not None:
        qr = time_rope(qr, ts, **rope)
        kr = time_rope(kr, ts, **rope)
    margs = dict(delay=delay, window=window, static_bidirectional=static_bidirectional,
                 global_tail=global_tail)
    rows = np.asarray(rows, np.int64)
    keys = np.asarray(keys, np.int64)
    need = np.zeros(L, bool)
    need[rows] = True
    for r0 in range(0, L, row_block):
        blk = np.arange(r0, min(L, r0 + row_block))
        need[blk] |= visible_rows(sk, ts, blk, cols=keys, **margs).any(axis=1)
    needed = np.nonzero(need)[0]
    lse = np.full(L, -np.inf)
    dsum = np.zeros(L)
    for r0 in range(0, needed.shape[0], row_block):
        blk = needed[r0:r0 + row_block]
        vis = visible_rows(sk, ts, blk, **margs)
        o_blk, lse[blk] = masked_softmax_attention(qr[blk], kr, vr, vis, scale)
        dsum[blk] = (gr[blk] * o_blk).sum(axis=1)

    def probs(blk, cols, vis):
        s = (qr[blk] @ kr[cols].T) * scale
        return np.where(vis, np.exp(s - lse[blk][:, None]), 0.0)

    allk = np.arange(L)
    vis = visible_rows(sk, ts, rows, **margs)
    p = probs(rows, allk, vis)
    ds = p * (gr[rows] @ vr.T - dsum[rows][:, None])
    dq = (ds @ kr) * scale
    dk = np.zeros((keys.shape[0], d))
    dv = np.zeros((keys.shape[0], d))
    for r0 in range(0, needed.shape[0], row_block):
        blk = needed[r0:r0 + row_block]
        visk = visible_rows(sk, ts, blk, cols=keys, **margs)
        pk = probs(blk, keys, visk)
        dv += pk.T @ gr[blk]
        dsk = pk * (gr[blk] @ vr[keys].T - dsum[blk][:, None])
        dk += (dsk.T @ qr[blk]) * scale
    if rope is not None:
        dq = time_rope_transpose(dq, ts[rows], **rope)
        dk = time_rope_transpose(dk, ts[keys], **rope)
    return dq, dk, dv


def qk_rmsnorm_backward(x: np.ndarray, gamma: Optional[np.ndarray], eps: float,
                        g: np.ndarray) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Gradients through QK Norm (qk_rmsnorm; TM20K section 2, SORT section
    3.3.2), float64.  For y = x * r * gamma with r = 1 / sqrt(mean(x^2) +
    eps) over the last axis (d) and upstream g = dLoss/dy, the chain rule
    (dr/dx_k = -r^3 x_k / d) gives
      dx = r * gamma * g - x * r^3 * sum_j(gamma_j g_j x_j) / d,
      dgamma = sum over every row of g * x * r   (None when gamma is None).
    """
    x = np.asarray(x, np.float64)
    g = np.asarray(g, np.float64)
    d = x.shape[-1]
    gam = np.ones(d) if gamma is None else np.asarray(gamma, np.float64)
    r = 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    t = (gam * g * x).sum(axis=-1, keepdims=True)
    dx = r * gam * g - x * r ** 3 * t / d
    dgamma = None if gamma is None else (g * x * r).reshape(-1, d).sum(axis=0)
    return dx, dgamma


def attention_backward_qk_norm(req_offsets, seg_kind, timestamps, q, k, v, do, *,
                               qk_norm: Dict, delay: int, window: int,
                               static_bidirectional: bool, rope=None, rope_times=None,
                               scale=None, global_tail: int = 0):
    """Gradients of the attention forward with QK Norm (attention_forward with
    qk_norm = dict(eps, gamma_q, gamma_k)): the masked attention backward
    at the normalised q, k (attention_backward, which also takes the
    gradients back through the rotation), then qk_rmsnorm_backward.  The
    gains are shared by every head, so their gradients sum over tokens and
    heads.  Returns (dq, dk, dv, dgamma_q, dgamma_k), float64."""
    eps = qk_norm["eps"]
    gq, gk = qk_norm.get("gamma_q"), qk_norm.get("gamma_k")
    qn = qk_rmsnorm(q, gq, eps)
    kn = qk_rmsnorm(k, gk, eps)
    dqn, dkn, dv = attention_backward(req_offsets, seg_kind, timestamps, qn, kn, v, do,
                                      delay=delay, window=window,
                                      static_bidirectional=static_bidirectional, rope=rope,
                                      rope_times=rope_times, scale=scale,
                                      global_tail=global_tail)
    dq, dgq = qk_rmsnorm_backward(q, gq, eps, dqn)
    dk, dgk = qk_rmsnorm_backward(k, gk, eps, dkn)
    return dq, dk, dv, dgq, dgk


# ---------------------------------------------------------------------------
# LazFormer history compression and per-layer pruning (section 2.3)
# ---------------------------------------------------------------------------

def compressed_history_length(L: int, keep: int, group: int) -> int:
    """Length after compression (eq. 16-18): the ell = min(L, keep) recent
    tokens plus N = ceil((L - ell) / group) group sums."""
    ell = min(L, keep)
    return ell + -(-(L - ell) // group)


def group_sum_compress(req_offsets, seg_kind, timestamps, x, *, keep: int, group: int):
    """Compress the HISTORY segment of every request (eq. 16-18).

    Per request with L history tokens in time order: the ell = min(L, keep)
    most recent are kept as they are; the L - ell older ones are summed in
    groups of `group`, counted back from the kept part, so a group with fewer
    members can only be the oldest one.  The output keeps time order:
    profile tokens, the group sums (oldest first), the kept history, then
    real-time and candidate tokens unchanged.  A group's timestamp is that of
    its newest member.  x: [T, ...] features (summed in float64).
    Returns (req_offsets, seg_kind, timestamps, y).
    """
    x = np.asarray(x, np.float64)
    offs, kinds, times, rows = [0], [], [], []
    for r in range(req_offsets.shape[0] - 1):
        a, b = int(req_offsets[r]), int(req_offsets[r + 1])
        hist = [j for j in range(a, b) if seg_kind[j] == HISTORY]
        ell = min(len(hist), keep)
        old = hist[:len(hist) - ell]
        # group boundaries counted back from the kept part
        groups = []
        end = len(old)
        while end > 0:
            start = max(0, end - group)
            groups.append(old[start:end])
            end = start
        groups.reverse()
        out = []
        for j in range(a, b):
            if seg_kind[j] == HISTORY:
                continue
            if seg_kind[j] == PROFILE:
                out.append((PROFILE, int(timestamps[j]), x[j]))
        for g in groups:
            out.append((HISTORY, int(timestamps[g[-1]]), x[g].sum(axis=0)))
        for j in hist[len(hist) - ell:]:
            out.append((HISTORY, int(timestamps[j]), x[j]))
        for j in range(a, b):
            if seg_kind[j] in (REALTIME, CANDIDATE):
                out.append((int(seg_kind[j]), int(timestamps[j]), x[j]))
        for kd, t, row in out:
            kinds.append(kd)
            times.append(t)
            rows.append(row)
        offs.append(offs[-1] + len(out))
    y = np.stack(rows) if rows else np.zeros((0,) + x.shape[1:])
    return (np.asarray(offs, np.int32), np.asarray(kinds, np.uint8),
            np.asarray(times, np.int64), y)


def pruned_history_length(l_tilde: int, n_min: int, layer: int, num_layers: int) -> int:
    """History positions layer `layer` (1-based) of `num_layers` keeps (eq. 22):
    min(L~, max(N_min, Round[L~ - (l - 1) / (L - 1) * (L~ - N_min)])), Round
    taking halves away from zero.  A single layer keeps L~."""
    if num_layers <= 1:
        return l_tilde
    val = l_tilde - (layer - 1) / (num_layers - 1) * (l_tilde - n_min)
    rnd = math.floor(abs(val) + 0.5) * (1 if val >= 0 else -1)
    return min(l_tilde, max(n_min, rnd))


def prune_history(req_offsets, seg_kind, timestamps, x, *, l_tilde, n_min: int, layer: int,
                  num_layers: int):
    """Input of layer `layer`: per request, the last N^l HISTORY tokens
    (N^l from eq. 22 with that request's L~ = l_tilde[r]) and every PROFILE,
    REALTIME and CANDIDATE token, in their order.  x: [T, ...].
    Returns (req_offsets, seg_kind, timestamps, y)."""
    x = np.asarray(x, np.float64)
    offs, sel = [0], []
    for r in range(req_offsets.shape[0] - 1):
        a, b = int(req_offsets[r]), int(req_offsets[r + 1])
        hist = [j for j in range(a, b) if seg_kind[j] == HISTORY]
        n = pruned_history_length(int(l_tilde[r]), n_min, layer, num_layers)
        drop = set(hist[:max(0, len(hist) - n)])
        keep = [j for j in range(a, b) if j not in drop]
        sel += keep
        offs.append(offs[-1] + len(keep))
    sel = np.asarray(sel, np.int64)
    return (np.asarray(offs, np.int32), seg_kind[sel].astype(np.uint8),
            timestamps[sel].astype(np.int64), x[sel])


def pruned_history_length_exp(l_tilde: int, n_min: int, decay: float, layer: int) -> int:
    """SORT's exponential query-pruning schedule (section 3.2.2, reading in
    the header): L~ * decay^(layer - 1) rounded half away from zero, at least
    N_min, at most L~."""
    val = l_tilde * decay ** (layer - 1)
    rnd = math.floor(abs(val) + 0.5) * (1 if val >= 0 else -1)
    return min(l_tilde, max(n_min, rnd))


def prune_history_keep(req_offsets, seg_kind, timestamps, x, *, keep):
    """Pruning to given lengths (any schedule, SORT section 3.2.2 without
    pooling): per request r, the last keep[r] HISTORY tokens and every
    PROFILE, REALTIME and CANDIDATE token, in their order.  x: [T, ...].
    Returns (req_offsets, seg_kind, timestamps, y)."""
    x = np.asarray(x, np.float64)
    offs, sel = [0], []
    for r in range(req_offsets.shape[0] - 1):
        a, b = int(req_offsets[r]), int(req_offsets[r + 1])
        hist = [j for j in range(a, b) if seg_kind[j] == HISTORY]
        drop = set(hist[:max(0, len(hist) - int(keep[r]))])
        kept = [j for j in range(a, b) if j not in drop]
        sel += kept
        offs.append(offs[-1] + len(kept))
    sel = np.asarray(sel, np.int64)
    return (np.asarray(offs, np.int32), seg_kind[sel].astype(np.uint8),
            timestamps[sel].astype(np.int64), x[sel])


def prune_history_pooled(req_offsets, seg_kind, timestamps, x, *, keep):
    """SORT's pooled query pruning (section 3.2.2, reading in the header):
    per request r, the history tokens beyond the last keep[r] are replaced by
    their mean, one HISTORY token placed where they were and dated as the
    newest of them; every other token is unchanged.  keep: [R] kept history
    lengths (from either schedule).  x: [T, ...].
    Returns (req_offsets, seg_kind, timestamps, y)."""
    x = np.asarray(x, np.float64)
    offs, kinds, times, rows = [0], [], [], []
    for r in range(req_offsets.shape[0] - 1):
        a, b = int(req_offsets[r]), int(req_offsets[r + 1])
        hist = [j for j in range(a, b) if seg_kind[j] == HISTORY]
        dropped = hist[:max(0, len(hist) - int(keep[r]))]
        n = 0
        for j in range(a, b):
            if j in dropped:
                if j == dropped[0]:
                    kinds.append(HISTORY)
                    times.append(int(timestamps[dropped[-1]]))
                    rows.append(x[dropped].mean(axis=0))
                    n += 1
                continue
            kinds.append(int(seg_kind[j]))
            times.append(int(timestamps[j]))
            rows.append(x[j])
            n += 1
        offs.append(offs[-1] + n)
    y = np.stack(rows) if rows else np.zeros((0,) + x.shape[1:])
    return (np.asarray(offs, np.int32), np.asarray(kinds, np.uint8),
            np.asarray(times, np.int64), y)


# ---------------------------------------------------------------------------
# Tile plan reference (128 query rows x 64 key columns)
# ---------------------------------------------------------------------------

def tile_plan_request(seg_kind, timestamps, *, delay, window, static_bidirectional,
                      tq: int = TILE_Q, tk: int = TILE_K, global_tail: int = 0):
    """Per-tile visible counts and classes of one request.

    Tile (qt, kt) covers request-local rows [tq*qt, tq*qt+tq) and columns
    [tk*kt, tk*kt+tk).  count = number of visible in-range cells.  FULL iff all
    tq*tk cells are in range and visible; EMPTY iff count == 0; PARTIAL
    otherwise.  Returns (count [nqt, nkt] int64, cls [nqt, nkt] uint8).
    """
    L = np.asarray(seg_kind).shape[0]
    nqt, nkt = -(-L // tq), -(-L // tk)
    count = np.zeros((nqt, nkt), np.int64)
    for qt in range(nqt):
        rows = np.arange(qt * tq, min(L, qt * tq + tq))
        vis = visible_rows(seg_kind, timestamps, rows, delay=delay, window=window,
                           static_bidirectional=static_bidirectional, global_tail=global_tail)
        padded = np.zeros((vis.shape[0], nkt * tk), dtype=bool)
        padded[:, :L] = vis
        count[qt] = padded.reshape(vis.shape[0], nkt, tk).sum(axis=(0, 2))
    cls = np.full((nqt, nkt), PARTIAL, np.uint8)
    cls[count == 0] = EMPTY
    cls[count == tq * tk] = FULL
    return count, cls


def tile_plan(req_offsets, seg_kind, timestamps, *, delay, window, static_bidirectional,
              tq: int = TILE_Q, tk: int = TILE_K, global_tail: int = 0) -> Dict[str, np.ndarray]:
    """Tile plan of a packed batch: flattened per-request tile arrays plus CSR.

    tile_count / tile_class: concatenation over requests of the row-major
    [nqt_r, nkt_r] arrays.  qtile_ptr / ktile_idx: CSR over all q-tiles in
    request order; each row lists its non-empty request-local k-tile indices in
    ascending order.  visible_pairs: total visible pairs (per head).
    """
    counts, classes, ptr, idx = [], [], [0], []
    for r in range(req_offsets.shape[0] - 1):
        a, b = int(req_offsets[r]), int(req_offsets[r + 1])
        c, k = tile_plan_request(seg_kind[a:b], timestamps[a:b], delay=delay, window=window,
                                 static_bidirectional=static_bidirectional, tq=tq, tk=tk,
                                 global_tail=global_tail)
        counts.append(c.ravel())
        classes.append(k.ravel())
        for qt in range(c.shape[0]):
            nz = np.nonzero(c[qt])[0]
            idx.append(nz)
            ptr.append(ptr[-1] + nz.shape[0])
    cat = lambda xs, dt: np.concatenate(xs).astype(dt) if xs else np.zeros(0, dt)
    tile_count = cat(counts, np.int64)
    return {
        "tile_count": tile_count,
        "tile_class": cat(classes, np.uint8),
        "qtile_ptr": np.asarray(ptr, np.int64),
        "ktile_idx": cat(idx, np.int64),
        "visible_pairs": int(tile_count.sum()),
    }
