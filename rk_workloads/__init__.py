"""Seeded synthetic inputs for request-centric masked attention.

This module only *draws inputs*: packed request layouts, per-token segment
kinds and integer timestamps, and Q/K/V values.  It holds none of the
method's arithmetic (no mask rule, no rotation, no attention) and is shared
by the CPU oracle's tests, the GPU parity tests and the benchmark so that all
of them see exactly the same bytes.

The five named workloads follow the shapes the pages describe:

* CADET (paper-daily.com, "CADET ..."): one sequence per user with
  impression/action events, a one-hour delay mask, candidates appended after
  the history ("how to score hundreds of candidates in 50 ms").
* SORT (10100.com article 149105610, section 3.1-3.2): request-centric
  samples, U2U causal with a sliding window, C2U full, C2C isolated.
* MTGR (joezjh.github.io blog index, "MTGR", model-structure part): profile +
  history mutually visible, a causal real-time sequence, targets that see
  only the real-time events before their own time.
* TM20K (liuzhao09.github.io, "TM20K", section 1.1): 20K-token histories with
  one target under full causal attention.

Timestamps are int64 Unix seconds.  "Log-uniform gaps" are
exp(U(ln 30 s, ln 21 d)).  Where a workload says its history spans one year,
the drawn gaps are rescaled so that the span is exactly 365 d (the CADET page
converts its one-year window with a factor of 365).  Values are rounded to
whole seconds with a minimum gap of one second.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

# Segment kinds, in the order they must appear inside a request.
PROFILE, HISTORY, REALTIME, CANDIDATE = 0, 1, 2, 3

NOW = 1_767_225_600          # 2026-01-01T00:00:00Z
YEAR = 31_536_000            # 365 days in seconds
DAY = 86_400
GAP_MIN = 30.0               # 30 s
GAP_MAX = 21.0 * DAY         # 21 days

# Time-RoPE constants from the CADET page (time-encoding section).
PHI_MIN = 1e-4
DT_MAX = float(YEAR)
BASE = 6e5


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16.
    Inputs must be finite.
    """
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    u = x.view(np.uint32)
    # finite values never overflow 32 bits here (largest is 0xFF7FFFFF + 0x8000)
    lsb = (u >> 16) & 1
    lsb += 0x7FFF
    u += lsb
    u &= 0xFFFF0000
    return x


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclass
class Workload:
    """One packed batch of requests plus the attention inputs."""

    name: str
    req_offsets: np.ndarray          # int32 [R+1]
    seg_kind: np.ndarray             # uint8 [T]
    timestamps: np.ndarray           # int64 [T]
    anchors: np.ndarray              # int64 [R]
    delay: int                       # seconds, 0 = off
    window: int                      # keys incl. self, 0 = off
    static_bidirectional: bool
    heads: int
    d_head: int
    dtype: str                       # "f32" or "bf16"
    q: Optional[np.ndarray] = None   # float32 [T, H, d], bf16-representable when dtype == "bf16"
    k: Optional[np.ndarray] = None
    v: Optional[np.ndarray] = None
    phi_min: float = PHI_MIN
    dt_max: float = DT_MAX
    base: float = BASE
    meta: dict = field(default_factory=dict)
    global_tail: int = 0             # LazFormer G: last G static positions exempt from the window

    @property
    def num_requests(self) -> int:
        return int(self.req_offsets.shape[0] - 1)

    @property
    def total_tokens(self) -> int:
        return int(self.req_offsets[-1])

    @property
    def n_candidates(self) -> int:
        return int(np.count_nonzero(self.seg_kind == CANDIDATE))

    def request(self, r: int) -> Tuple[int, int]:
        return int(self.req_offsets[r]), int(self.req_offsets[r + 1])


def _log_uniform_gaps(rng: np.random.Generator, n: int) -> np.ndarray:
    return np.exp(rng.uniform(np.log(GAP_MIN), np.log(GAP_MAX), size=n))


def _int_gaps(g: np.ndarray) -> np.ndarray:
    return np.maximum(1, np.rint(g)).astype(np.int64)


def history_raw(rng: np.random.Generator, n: int, end: int) -> np.ndarray:
    """n sorted timestamps ending at `end` with raw log-uniform gaps."""
    if n == 0:
        return np.zeros(0, np.int64)
    gi = _int_gaps(_log_uniform_gaps(rng, n - 1))
    back = np.concatenate([np.cumsum(gi[::-1])[::-1], [0]])
    return (end - back).astype(np.int64)


def history_span(rng: np.random.Generator, n: int, end: int, span: int = YEAR) -> np.ndarray:
    """n sorted timestamps ending at `end` whose first-to-last span is exactly `span`."""
    if n == 0:
        return np.zeros(0, np.int64)
    if n == 1:
        return np.array([end], np.int64)
    g = _log_uniform_gaps(rng, n - 1)
    gi = _int_gaps(g * (span / g.sum()))
    gi[np.argmax(gi)] += span - int(gi.sum())
    assert gi.min() >= 1 and int(gi.sum()) == span
    t = np.concatenate([[0], np.cumsum(gi)]) + (end - span)
    return t.astype(np.int64)


def pack(requests: Sequence[Sequence[Tuple[int, np.ndarray]]]) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Pack requests given as lists of (segment kind, timestamps) into flat arrays."""
    offs = [0]
    kinds: List[np.ndarray] = []
    times: List[np.ndarray] = []
    for segs in requests:
        n = 0
        for kind, ts in segs:
            ts = np.asarray(ts, np.int64)
            kinds.append(np.full(ts.shape[0], kind, np.uint8))
            times.append(ts)
            n += ts.shape[0]
        offs.append(offs[-1] + n)
    seg = np.concatenate(kinds) if kinds else np.zeros(0, np.uint8)
    ts = np.concatenate(times) if times else np.zeros(0, np.int64)
    return np.asarray(offs, np.int32), seg, ts


def draw_qkv(rng: np.random.Generator, T: int, H: int, d: int, dtype: str):
    q = rng.standard_normal((T, H, d), dtype=np.float32)
    k = rng.standard_normal((T, H, d), dtype=np.float32)
    v = rng.standard_normal((T, H, d), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    return q, k, v


def draw_grad(wl: "Workload", seed: Optional[int] = None) -> np.ndarray:
    """Upstream gradient dO ~ N(0, 1) of shape [T, H, d] for backward tests and
    the backward benchmark; bf16-rounded for bf16 workloads.  Drawn from its
    own generator (seed: the workload's seed + 7919 unless given), so the
    forward inputs are unchanged."""
    if seed is None:
        seed = int(wl.meta.get("seed", 0)) + 7919
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((wl.total_tokens, wl.heads, wl.d_head), dtype=np.float32)
    return bf16_round(g) if wl.dtype == "bf16" else g


CONFIG_NAMES = {
    1: "tiny-f32-cadet-1x(256+16)",
    2: "cadet-64x1024-delay1h",
    3: "serving-32x(2048+512)-w256",
    4: "mtgr-16x(32+3000+200+100)",
    5: "tm20k-8x(20000+1)-causal",
}


def make_config(n: int, with_qkv: bool = True) -> Workload:
    """Build one of the five named workloads with seed 1000 + n."""
    rng = np.random.default_rng(1000 + n)
    requests = []
    if n == 1:
        requests.append([(HISTORY, history_raw(rng, 256, NOW)),
                         (CANDIDATE, np.full(16, NOW, np.int64))])
        H, d, dtype, delay, window, bidir = 2, 32, "f32", 3600, 0, False
    elif n == 2:
        for _ in range(64):
            requests.append([(HISTORY, history_span(rng, 1024, NOW))])
        H, d, dtype, delay, window, bidir = 4, 64, "bf16", 3600, 0, False
    elif n == 3:
        for _ in range(32):
            requests.append([(HISTORY, history_span(rng, 2048, NOW - 60)),
                             (CANDIDATE, np.full(512, NOW, np.int64))])
        H, d, dtype, delay, window, bidir = 8, 64, "bf16", 0, 256, False
    elif n == 4:
        for _ in range(16):
            picks = rng.choice(DAY, size=300, replace=False).astype(np.int64) + (NOW - DAY + 1)
            requests.append([(PROFILE, np.full(32, NOW, np.int64)),
                             (HISTORY, history_span(rng, 3000, NOW - DAY)),
                             (REALTIME, np.sort(picks[:200])),
                             (CANDIDATE, picks[200:])])
        H, d, dtype, delay, window, bidir = 8, 64, "bf16", 0, 0, True
    elif n == 5:
        for _ in range(8):
            requests.append([(HISTORY, history_span(rng, 20000, NOW - 60)),
                             (CANDIDATE, np.array([NOW], np.int64))])
        H, d, dtype, delay, window, bidir = 8, 64, "bf16", 0, 0, False
    else:
        raise ValueError(f"unknown workload {n}")
    offs, seg, ts = pack(requests)
    R = offs.shape[0] - 1
    wl = Workload(name=CONFIG_NAMES[n], req_offsets=offs, seg_kind=seg, timestamps=ts,
                  anchors=np.full(R, NOW, np.int64), delay=delay, window=window,
                  static_bidirectional=bidir, heads=H, d_head=d, dtype=dtype,
                  meta={"config": n, "seed": 1000 + n})
    if n == 2:
        # impression/action alternation: generator metadata only, never passed to the library
        wl.meta["token_role"] = np.tile(np.array([0, 1], np.uint8), seg.shape[0] // 2)
    if with_qkv:
        wl.q, wl.k, wl.v = draw_qkv(rng, seg.shape[0], H, d, dtype)
    return wl


def make_custom(requests: Sequence[Sequence[Tuple[int, np.ndarray]]], *, heads: int, d_head: int,
                dtype: str = "f32", delay: int = 0, window: int = 0,
                static_bidirectional: bool = False, seed: int = 0,
                anchors: Optional[np.ndarray] = None, with_qkv: bool = True,
                name: str = "custom", global_tail: int = 0) -> Workload:
    """Build a workload from an explicit request layout (tests, edge cases)."""
    offs, seg, ts = pack(requests)
    R = offs.shape[0] - 1
    if anchors is None:
        anchors = np.full(R, NOW, np.int64)
    wl = Workload(name=name, req_offsets=offs, seg_kind=seg, timestamps=ts,
                  anchors=np.asarray(anchors, np.int64), delay=delay, window=window,
                  static_bidirectional=static_bidirectional, heads=heads, d_head=d_head,
                  dtype=dtype, meta={"seed": seed}, global_tail=global_tail)
    if with_qkv:
        rng = np.random.default_rng(seed)
        wl.q, wl.k, wl.v = draw_qkv(rng, seg.shape[0], heads, d_head, dtype)
    return wl


def random_layout(rng: np.random.Generator, n_requests: int, max_len: int, *,
                  kinds=(PROFILE, HISTORY, REALTIME, CANDIDATE), allow_empty: bool = True):
    """Random ragged requests (segment lengths may be zero) for edge-case tests.

    Profile tokens are dated, per request: at the anchor NOW (the pages give
    profile tokens no time; half of the requests), at the earliest history
    timestamp (a quarter), or at sorted times up to 30 days before the
    earliest history timestamp (a quarter).  Every choice keeps PROFILE and
    HISTORY each in time order.  Real-time events are sorted; candidate
    times are in random order.
    """
    reqs = []
    for _ in range(n_requests):
        budget = int(rng.integers(0 if allow_empty else 1, max_len + 1))
        cuts = np.sort(rng.integers(0, budget + 1, size=len(kinds) - 1))
        lens = dict(zip(kinds, (int(x) for x in np.diff(np.concatenate([[0], cuts, [budget]])))))
        hist = history_raw(rng, lens.get(HISTORY, 0), NOW - DAY)
        t_first = int(hist[0]) if hist.shape[0] else NOW - DAY
        prof_mode = int(rng.integers(0, 4))
        segs = []
        for kind in kinds:
            n = lens[kind]
            if kind == PROFILE:
                if prof_mode < 2:
                    ts = np.full(n, NOW, np.int64)
                elif prof_mode == 2:
                    ts = np.full(n, t_first, np.int64)
                else:
                    ts = np.sort(rng.integers(t_first - 30 * DAY, t_first + 1, size=n)).astype(np.int64)
            elif kind == HISTORY:
                ts = hist
            elif kind == REALTIME:
                ts = np.sort(rng.integers(NOW - DAY + 1, NOW + 1, size=n)).astype(np.int64)
            else:
                ts = rng.integers(NOW - DAY + 1, NOW + 1, size=n).astype(np.int64)
            segs.append((kind, ts))
        reqs.append(segs)
    return reqs
