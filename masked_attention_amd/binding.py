"""Thin Python binding over librk's C ABI (include/rk.h).

Argument marshalling only: torch tensors supply device memory and the
current HIP stream; every step of the computation runs in librk's kernels.
Names follow the C entry points.
"""

from __future__ import annotations

import ctypes as C
from typing import Optional

import numpy as np
import torch

from . import _rk
from ._rk import check, lib, sized


def _stream(stream: Optional[torch.cuda.Stream]) -> C.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return _rk.RK_F32
    if t.dtype == torch.bfloat16:
        return _rk.RK_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def rope_params(phi_min: float, dt_max: float, base: float, kinds: int = 0) -> _rk.rk_rope_params:
    return sized(_rk.rk_rope_params, phi_min=float(phi_min), dt_max=float(dt_max),
                 base=float(base), kinds=int(kinds))


class Batch:
    """Device copies of one packed batch plus its rk_batch descriptor."""

    def __init__(self, req_offsets, seg_kind, timestamps, anchors, device="cuda"):
        self.req_offsets_host = np.ascontiguousarray(req_offsets, dtype=np.int32)
        self.R = int(self.req_offsets_host.shape[0] - 1)
        self.T = int(self.req_offsets_host[-1])
        self.req_offsets = torch.from_numpy(self.req_offsets_host.copy()).to(device)
        self.seg_kind = torch.from_numpy(np.ascontiguousarray(seg_kind, dtype=np.uint8)).to(device)
        self.timestamps = torch.from_numpy(np.ascontiguousarray(timestamps, dtype=np.int64)).to(device)
        self.anchors = torch.from_numpy(np.ascontiguousarray(anchors, dtype=np.int64)).to(device)
        self.c = sized(_rk.rk_batch, num_requests=self.R, total_tokens=self.T,
                       req_offsets_host=self.req_offsets_host.ctypes.data,
                       req_offsets_dev=self.req_offsets.data_ptr(),
                       seg_kind_dev=self.seg_kind.data_ptr(),
                       timestamps_dev=self.timestamps.data_ptr(),
                       anchors_dev=self.anchors.data_ptr())

    @classmethod
    def from_workload(cls, wl, device="cuda") -> "Batch":
        return cls(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.anchors, device=device)


def rk_plan_workspace_size(batch: Batch, num_heads: int) -> int:
    n = C.c_size_t()
    check(lib().rk_plan_workspace_size(C.byref(batch.c), int(num_heads), C.byref(n)),
          "rk_plan_workspace_size")
    return int(n.value)


class Plan:
    """A tile plan built by rk_mask_plan in a torch-owned workspace."""

    def __init__(self, batch: Batch, *, delay: int = 0, window: int = 0,
                 static_bidirectional: bool = False, num_heads: int = 1,
                 candidates_only: bool = False, global_tail: int = 0, backward: bool = False,
                 stream: Optional[torch.cuda.Stream] = None,
                 workspace: Optional[torch.Tensor] = None):
        self.batch = batch
        self.num_heads = int(num_heads)
        size = rk_plan_workspace_size(batch, num_heads)
        if workspace is None:
            workspace = torch.empty(max(size, 256), dtype=torch.uint8, device=batch.seg_kind.device)
        self.workspace = workspace
        flags = (_rk.RK_STATIC_BIDIRECTIONAL if static_bidirectional else 0) | (
            _rk.RK_QUERY_CANDIDATES_ONLY if candidates_only else 0) | (
            _rk.RK_PLAN_BACKWARD if backward else 0)
        self.params = sized(_rk.rk_mask_params, delay=int(delay), window=int(window),
                            global_tail=int(global_tail), flags=flags)
        h = C.c_void_p()
        check(lib().rk_mask_plan(C.byref(batch.c), C.byref(self.params), self.num_heads,
                                 C.c_void_p(workspace.data_ptr()),
                                 C.c_size_t(workspace.numel()), C.byref(h), _stream(stream)),
              "rk_mask_plan")
        self.handle = h
        info = sized(_rk.rk_plan_info)
        check(lib().rk_plan_get_info(h, C.byref(info)), "rk_plan_get_info")
        self.info = info

    # -- views into the workspace (valid after the stream ran the planner)
    def _view(self, off: int, n: int, dtype: torch.dtype) -> torch.Tensor:
        nbytes = n * torch.empty(0, dtype=dtype).element_size()
        return self.workspace[off:off + nbytes].view(dtype)

    @property
    def num_tiles(self) -> int:
        return int(self.info.num_tiles)

    @property
    def num_qtiles(self) -> int:
        return int(self.info.num_qtiles)

    def tile_class(self) -> torch.Tensor:
        return self._view(self.info.off_tile_class, self.num_tiles, torch.uint8)

    def tile_count(self) -> torch.Tensor:
        return self._view(self.info.off_tile_count, self.num_tiles, torch.int32)

    def qtile_ptr(self) -> torch.Tensor:
        return self._view(self.info.off_qtile_ptr, self.num_qtiles + 1, torch.int32)

    def ktile_idx(self) -> torch.Tensor:
        n = int(self.qtile_ptr()[-1].item()) if self.num_qtiles else 0
        return self._view(self.info.off_ktile_idx, n, torch.int32)

    def row_desc(self) -> torch.Tensor:
        return self._view(self.info.off_row_desc, 2 * self.batch.T, torch.int32).view(-1, 2)

    def sched(self) -> torch.Tensor:
        return self._view(self.info.off_sched, int(self.info.num_sched_slots), torch.int32)

    def work(self) -> Optional[torch.Tensor]:
        """Work list [slots, 4] = (item, first, end, part), or None."""
        n = int(self.info.num_work_slots)
        if n == 0:
            return None
        return self._view(self.info.off_work, 4 * n, torch.int32).view(n, 4)

    def splits(self) -> Optional[torch.Tensor]:
        """Split items [RK_SPLIT_SLOTS, 4] = (item, first part, parts, 0), or None."""
        if int(self.info.num_work_slots) == 0:
            return None
        n = _rk.RK_SPLIT_SLOTS
        return self._view(self.info.off_splits, 4 * n, torch.int32).view(n, 4)

    @property
    def num_kblocks(self) -> int:
        """Key blocks of 128 keys (the backward's key-major items)."""
        return int(self.info.num_kblocks)

    def kt_ptr(self) -> Optional[torch.Tensor]:
        """Key-major CSR row pointers [num_kblocks + 1] (backward plans), or None."""
        if int(self.info.num_ksched_slots) == 0:
            return None
        return self._view(self.info.off_kt_ptr, self.num_kblocks + 1, torch.int32)

    def qtile_word(self) -> Optional[torch.Tensor]:
        """Key-major CSR entries: request-local q-tile | (PARTIAL << 31), or None."""
        ptr = self.kt_ptr()
        if ptr is None:
            return None
        n = int(ptr[-1].item()) if self.num_kblocks else 0
        return self._view(self.info.off_qtile_word, n, torch.int32)

    def ksched(self) -> Optional[torch.Tensor]:
        n = int(self.info.num_ksched_slots)
        if n == 0:
            return None
        return self._view(self.info.off_ksched, n, torch.int32)

    def stats(self, stream: Optional[torch.cuda.Stream] = None, raise_on_error: bool = True) -> dict:
        t = sized(_rk.rk_plan_totals)
        st = lib().rk_plan_stats(self.handle, C.byref(t), _stream(stream))
        if st not in (_rk.RK_OK, _rk.RK_ERR_SEGMENT_ORDER, _rk.RK_ERR_UNSORTED_TIME) or (
                raise_on_error and st != _rk.RK_OK):
            check(st, "rk_plan_stats")
        return {"status": st, "device_errors": int(t.device_errors),
                "visible_pairs": int(t.visible_pairs), "full_tiles": int(t.full_tiles),
                "partial_tiles": int(t.partial_tiles), "empty_tiles": int(t.empty_tiles),
                "work_entries": int(t.work_entries), "split_items": int(t.split_items)}

    def close(self) -> None:
        if getattr(self, "handle", None) is not None and self.handle.value:
            torch.cuda.synchronize()
            lib().rk_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def rk_mask_plan(batch: Batch, **kw) -> Plan:
    return Plan(batch, **kw)


def rk_time_rope(batch: Batch, x: torch.Tensor, *, phi_min: float, dt_max: float, base: float,
                 out: Optional[torch.Tensor] = None, kinds=None,
                 stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Rotate x [T, H, d] (d contiguous) by time RoPE into out (default: new tensor).

    kinds: None (every token) or an iterable of segment kinds (RK_SEG_*): only
    tokens of those kinds are rotated, the other rows of out are left as they
    were (so out should be given)."""
    if x.dim() != 3 or x.stride(2) != 1:
        raise ValueError("x must be [T, H, d] with d contiguous")
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    mask = 0 if kinds is None else sum(1 << int(k) for k in set(kinds))
    rp = rope_params(phi_min, dt_max, base, kinds=mask)
    check(lib().rk_time_rope(C.byref(batch.c), C.byref(rp), C.c_void_p(x.data_ptr()),
                             C.c_void_p(out.data_ptr()), _dtype_code(x), x.shape[1], x.shape[2],
                             x.stride(0), x.stride(1), out.stride(0), out.stride(1), _stream(stream)),
          "rk_time_rope")
    return out


def qk_norm_params(eps: float, gamma_q: Optional[torch.Tensor] = None,
                   gamma_k: Optional[torch.Tensor] = None) -> _rk.rk_qk_norm_params:
    """QK Norm parameters; gains are fp32 device tensors [d_head] (kept alive by
    the caller) or None."""
    for g in (gamma_q, gamma_k):
        if g is not None and (g.dtype != torch.float32 or not g.is_contiguous()):
            raise ValueError("QK Norm gains must be contiguous float32 tensors")
    return sized(_rk.rk_qk_norm_params, eps=float(eps),
                 gamma_q=gamma_q.data_ptr() if gamma_q is not None else None,
                 gamma_k=gamma_k.data_ptr() if gamma_k is not None else None)


def rk_qk_norm_rope(batch: Batch, x: torch.Tensor, *, eps: float,
                    gamma: Optional[torch.Tensor] = None, rope: Optional[dict] = None,
                    out: Optional[torch.Tensor] = None, kinds=None,
                    stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """QK Norm (then time RoPE when rope is given) of x [T, H, d] into out."""
    if x.dim() != 3 or x.stride(2) != 1:
        raise ValueError("x must be [T, H, d] with d contiguous")
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    mask = 0 if kinds is None else sum(1 << int(k) for k in set(kinds))
    rp = rope_params(**rope, kinds=mask) if rope is not None else None
    if gamma is not None and (gamma.dtype != torch.float32 or not gamma.is_contiguous()):
        raise ValueError("gamma must be a contiguous float32 tensor")
    check(lib().rk_qk_norm_rope(C.byref(batch.c), C.byref(rp) if rp is not None else None,
                                float(eps), C.c_void_p(gamma.data_ptr() if gamma is not None else 0),
                                C.c_void_p(x.data_ptr()), C.c_void_p(out.data_ptr()),
                                _dtype_code(x), x.shape[1], x.shape[2], x.stride(0), x.stride(1),
                                out.stride(0), out.stride(1), _stream(stream)), "rk_qk_norm_rope")
    return out


def _attn_args(plan: Plan, q, k, v, o, lse, scale, rope, reference, workspace,
               k_prerotated=False, qk_norm=None):
    for t in (q, k, v, o):
        if t.dim() != 3 or t.stride(2) != 1:
            raise ValueError("q, k, v, o must be [T, H, d] with d contiguous")
    flags = (_rk.RK_ATTN_REFERENCE_KERNEL if reference else 0) | (
        _rk.RK_ATTN_K_PREROTATED if k_prerotated else 0)
    a = sized(_rk.rk_attn_args, flags=flags,
              dtype=_dtype_code(q), num_heads=q.shape[1], d_head=q.shape[2],
              q=q.data_ptr(), k=k.data_ptr(), v=v.data_ptr(), o=o.data_ptr(),
              lse=lse.data_ptr() if lse is not None else None,
              q_stride_tok=q.stride(0), q_stride_head=q.stride(1),
              k_stride_tok=k.stride(0), k_stride_head=k.stride(1),
              v_stride_tok=v.stride(0), v_stride_head=v.stride(1),
              o_stride_tok=o.stride(0), o_stride_head=o.stride(1),
              scale=float(scale))
    if rope is not None:
        a.rope = C.cast(C.pointer(rope), C.c_void_p)
    if qk_norm is not None:
        a.qk_norm = C.cast(C.pointer(qk_norm), C.c_void_p)
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    return a


def rk_attn_workspace_size(plan: Plan, q, k, v, *, rope=None, reference=False,
                           k_prerotated=False) -> int:
    o = q  # only shapes/strides are read
    rp = rope_params(**rope) if rope is not None else None
    a = _attn_args(plan, q, k, v, o, None, 0.0, rp, reference, None, k_prerotated)
    n = C.c_size_t()
    check(lib().rk_attn_workspace_size(plan.handle, C.byref(a), C.byref(n)), "rk_attn_workspace_size")
    return int(n.value)


def rk_masked_attn_fwd(plan: Plan, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
                       out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                       want_lse: bool = False, scale: float = 0.0, rope: Optional[dict] = None,
                       reference: bool = False, workspace: Optional[torch.Tensor] = None,
                       k_prerotated: bool = False, qk_norm: Optional[dict] = None,
                       stream: Optional[torch.cuda.Stream] = None):
    """Masked attention forward over `plan`.  Returns (o, lse or None).

    qk_norm: None, or dict(eps=..., gamma_q=tensor or None, gamma_k=tensor or
    None): QK Norm of Q and K before the rotation.

    rope: None, or dict(phi_min=..., dt_max=..., base=...) to rotate Q and K
    by time RoPE with the plan's timestamps and anchors.  k_prerotated:
    K already holds rk_time_rope's output; only Q is rotated.
    """
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None and want_lse:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    rp = rope_params(**rope) if rope is not None else None
    nq = qk_norm_params(**qk_norm) if qk_norm is not None else None
    a = _attn_args(plan, q, k, v, out, lse, scale, rp, reference, workspace, k_prerotated, nq)
    n = C.c_size_t()
    check(lib().rk_attn_workspace_size(plan.handle, C.byref(a), C.byref(n)), "rk_attn_workspace_size")
    if n.value and workspace is None:
        workspace = torch.empty(n.value, dtype=torch.uint8, device=q.device)
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = n.value
    check(lib().rk_masked_attn_fwd(plan.handle, C.byref(a), _stream(stream)), "rk_masked_attn_fwd")
    # keep the workspace alive until the caller synchronises
    out._rk_workspace = workspace  # type: ignore[attr-defined]
    return out, lse


def rk_masked_attn_fwd_noalloc(plan: Plan, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
                               out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                               scale: float = 0.0, rope: Optional[dict] = None,
                               reference: bool = False, k_prerotated: bool = False,
                               qk_norm: Optional[dict] = None,
                               stream: Optional[torch.cuda.Stream] = None):
    """rk_masked_attn_fwd with the library's per-GPU scratch array in place of
    a workspace: nothing is allocated, so `out` (and `lse`, if wanted) come
    from the caller.  Returns (out, lse)."""
    rp = rope_params(**rope) if rope is not None else None
    nq = qk_norm_params(**qk_norm) if qk_norm is not None else None
    a = _attn_args(plan, q, k, v, out, lse, scale, rp, reference, None, k_prerotated, nq)
    check(lib().rk_masked_attn_fwd_noalloc(plan.handle, C.byref(a), _stream(stream)),
          "rk_masked_attn_fwd_noalloc")
    return out, lse


def _bwd_args(q, k, v, o, do, lse, dq, dk, dv, scale, rope, reference, k_prerotated, workspace):
    for t in (q, k, v, o, do, dq, dk, dv):
        if t.dim() != 3 or t.stride(2) != 1:
            raise ValueError("q, k, v, o, do, dq, dk, dv must be [T, H, d] with d contiguous")
    flags = (_rk.RK_ATTN_REFERENCE_KERNEL if reference else 0) | (
        _rk.RK_ATTN_K_PREROTATED if k_prerotated else 0)
    a = sized(_rk.rk_attn_bwd_args, flags=flags, dtype=_dtype_code(q), num_heads=q.shape[1],
              d_head=q.shape[2], q=q.data_ptr(), k=k.data_ptr(), v=v.data_ptr(),
              o=o.data_ptr(), d_o=do.data_ptr(), lse=lse.data_ptr() if lse is not None else None,
              dq=dq.data_ptr(), dk=dk.data_ptr(), dv=dv.data_ptr(),
              q_stride_tok=q.stride(0), q_stride_head=q.stride(1),
              k_stride_tok=k.stride(0), k_stride_head=k.stride(1),
              v_stride_tok=v.stride(0), v_stride_head=v.stride(1),
              o_stride_tok=o.stride(0), o_stride_head=o.stride(1),
              do_stride_tok=do.stride(0), do_stride_head=do.stride(1),
              dq_stride_tok=dq.stride(0), dq_stride_head=dq.stride(1),
              dk_stride_tok=dk.stride(0), dk_stride_head=dk.stride(1),
              dv_stride_tok=dv.stride(0), dv_stride_head=dv.stride(1),
              scale=float(scale))
    if rope is not None:
        a.rope = C.cast(C.pointer(rope), C.c_void_p)
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    return a


def rk_masked_attn_bwd(plan: Plan, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       o: torch.Tensor, lse: torch.Tensor, do: torch.Tensor, *,
                       dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                       dv: Optional[torch.Tensor] = None, scale: float = 0.0,
                       rope: Optional[dict] = None, reference: bool = False,
                       k_prerotated: bool = False, workspace: Optional[torch.Tensor] = None,
                       qk_norm: Optional[dict] = None,
                       stream: Optional[torch.cuda.Stream] = None):
    """Gradients (dq, dk, dv) of the masked attention forward over `plan`
    (built with backward=True), given the forward's o and lse and the
    upstream gradient do.  q, k, v, scale, rope, k_prerotated and qk_norm
    (dict(eps=..., gamma_q=tensor or None, gamma_k=tensor or None)) are
    those of the forward call.  With qk_norm the result is (dq, dk, dv,
    dgamma_q, dgamma_k), the gains' gradients as fp32 [d] tensors (None for
    an absent gain)."""
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    rp = rope_params(**rope) if rope is not None else None
    a = _bwd_args(q, k, v, o, do, lse, dq, dk, dv, scale, rp, reference, k_prerotated, workspace)
    nq, dgq, dgk = None, None, None
    if qk_norm is not None:
        nq = qk_norm_params(**qk_norm)
        a.qk_norm = C.cast(C.pointer(nq), C.c_void_p)
        d = q.shape[2]
        if qk_norm.get("gamma_q") is not None:
            dgq = torch.empty(d, dtype=torch.float32, device=q.device)
            a.dgamma_q = dgq.data_ptr()
        if qk_norm.get("gamma_k") is not None:
            dgk = torch.empty(d, dtype=torch.float32, device=q.device)
            a.dgamma_k = dgk.data_ptr()
    n = C.c_size_t()
    check(lib().rk_attn_bwd_workspace_size(plan.handle, C.byref(a), C.byref(n)),
          "rk_attn_bwd_workspace_size")
    if n.value and workspace is None:
        workspace = torch.empty(n.value, dtype=torch.uint8, device=q.device)
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = n.value
    check(lib().rk_masked_attn_bwd(plan.handle, C.byref(a), _stream(stream)), "rk_masked_attn_bwd")
    dq._rk_workspace = workspace  # type: ignore[attr-defined]
    if qk_norm is not None:
        return dq, dk, dv, dgq, dgk
    return dq, dk, dv


def rk_pointwise_attn_fwd(plan: Plan, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
                          out: Optional[torch.Tensor] = None, scale: float = 0.0,
                          pos_bias: Optional[torch.Tensor] = None,
                          time_bias: Optional[torch.Tensor] = None, reference: bool = False,
                          stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """HSTU pointwise attention over `plan`: O_i = sum over visible j of
    SiLU(scale q_i . k_j + rab_ij) v_j (scale 0 = 1).  pos_bias / time_bias:
    float32 device tensors (the rab tables, shared by every head) or None."""
    for t in (q, k, v):
        if t.dim() != 3 or t.stride(2) != 1:
            raise ValueError("q, k, v must be [T, H, d] with d contiguous")
    for t in (pos_bias, time_bias):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("bias tables must be contiguous float32 tensors")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    a = sized(_rk.rk_pointwise_args, flags=_rk.RK_ATTN_REFERENCE_KERNEL if reference else 0,
              dtype=_dtype_code(q), num_heads=q.shape[1], d_head=q.shape[2],
              q=q.data_ptr(), k=k.data_ptr(), v=v.data_ptr(), o=out.data_ptr(),
              q_stride_tok=q.stride(0), q_stride_head=q.stride(1),
              k_stride_tok=k.stride(0), k_stride_head=k.stride(1),
              v_stride_tok=v.stride(0), v_stride_head=v.stride(1),
              o_stride_tok=out.stride(0), o_stride_head=out.stride(1), scale=float(scale),
              num_pos_buckets=pos_bias.numel() if pos_bias is not None else 0,
              num_time_buckets=time_bias.numel() if time_bias is not None else 0,
              pos_bias=pos_bias.data_ptr() if pos_bias is not None else None,
              time_bias=time_bias.data_ptr() if time_bias is not None else None)
    check(lib().rk_pointwise_attn_fwd(plan.handle, C.byref(a), _stream(stream)),
          "rk_pointwise_attn_fwd")
    return out


# ---- LazFormer pre-passes -------------------------------------------------

class Layout:
    """Host copy of a packed layout (numpy arrays) as passed to and returned
    by the layout functions; `ranges` [T, 2] describes each token as input
    rows [b, e) of the layout it came from (None for an original layout)."""

    def __init__(self, req_offsets, seg_kind, timestamps, ranges=None):
        self.req_offsets = np.ascontiguousarray(req_offsets, dtype=np.int32)
        self.seg_kind = np.ascontiguousarray(seg_kind, dtype=np.uint8)
        self.timestamps = np.ascontiguousarray(timestamps, dtype=np.int64)
        self.ranges = ranges
        self.R = int(self.req_offsets.shape[0] - 1)
        self.T = int(self.req_offsets[-1]) if self.R >= 0 else 0

    @classmethod
    def from_workload(cls, wl) -> "Layout":
        return cls(wl.req_offsets, wl.seg_kind, wl.timestamps)

    def c(self) -> _rk.rk_host_layout:
        return sized(_rk.rk_host_layout, num_requests=self.R, total_tokens=self.T,
                     req_offsets=self.req_offsets.ctypes.data,
                     seg_kind=self.seg_kind.ctypes.data if self.T else None,
                     timestamps=self.timestamps.ctypes.data if self.T else None)

    def history_lengths(self) -> np.ndarray:
        """HISTORY tokens of each request."""
        idx = np.repeat(np.arange(self.R), np.diff(self.req_offsets))
        return np.bincount(idx[self.seg_kind == _rk.RK_SEG_HISTORY],
                           minlength=self.R).astype(np.int32)


def _layout_call(fn, lay: Layout, *args) -> Layout:
    inc = lay.c()
    out = sized(_rk.rk_layout_out, capacity=0)
    offs = np.zeros(lay.R + 1, np.int32)
    out.req_offsets = offs.ctypes.data
    st = fn(C.byref(inc), *args, C.byref(out))
    if st == _rk.RK_ERR_WORKSPACE_TOO_SMALL:
        n = int(out.total_tokens)
        kinds = np.zeros(n, np.uint8)
        times = np.zeros(n, np.int64)
        ranges = np.zeros((n, 2), np.int32)
        out = sized(_rk.rk_layout_out, capacity=n, req_offsets=offs.ctypes.data,
                    seg_kind=kinds.ctypes.data, timestamps=times.ctypes.data,
                    ranges=ranges.ctypes.data)
        st = fn(C.byref(inc), *args, C.byref(out))
    else:
        kinds, times, ranges = (np.zeros(0, np.uint8), np.zeros(0, np.int64),
                                np.zeros((0, 2), np.int32))
    check(st, fn.__name__)
    return Layout(offs, kinds, times, ranges)


def rk_compress_layout(lay: Layout, *, keep: int, group: int) -> Layout:
    """LazFormer group-sum compression layout (eq. 16-18)."""
    return _layout_call(lib().rk_compress_layout, lay, int(keep), int(group))


def rk_pruned_history_length(l_tilde: int, n_min: int, layer: int, num_layers: int) -> int:
    n = C.c_int32()
    check(lib().rk_pruned_history_length(int(l_tilde), int(n_min), int(layer), int(num_layers),
                                         C.byref(n)), "rk_pruned_history_length")
    return int(n.value)


def rk_prune_layout(lay: Layout, *, l_tilde, n_min: int, layer: int, num_layers: int) -> Layout:
    """Layer input layout after pruning to the last N^l history tokens (eq. 22)."""
    lt = np.ascontiguousarray(l_tilde, dtype=np.int32)
    return _layout_call(lib().rk_prune_layout, lay, C.c_void_p(lt.ctypes.data), int(n_min),
                        int(layer), int(num_layers))


def prune_params(*, schedule: str = "linear", n_min: int, layer: int, num_layers: int = 1,
                 decay: float = 1.0, pool: bool = False) -> _rk.rk_prune_params:
    """SORT query pruning parameters: schedule "linear" (LazFormer eq. 22)
    or "exp" (decay^(layer - 1)); pool: the pruned history becomes one
    mean-pooled token."""
    code = {"linear": _rk.RK_PRUNE_LINEAR, "exp": _rk.RK_PRUNE_EXP}[schedule]
    return sized(_rk.rk_prune_params, schedule=code, n_min=int(n_min), layer=int(layer),
                 num_layers=int(num_layers), pool=1 if pool else 0, decay=float(decay))


def rk_pruned_history_length_ex(l_tilde: int, **params) -> int:
    p = prune_params(**params)
    n = C.c_int32()
    check(lib().rk_pruned_history_length_ex(int(l_tilde), C.byref(p), C.byref(n)),
          "rk_pruned_history_length_ex")
    return int(n.value)


def rk_prune_layout_ex(lay: Layout, *, l_tilde, **params) -> Layout:
    """Layer input layout of SORT's query pruning (linear or exponential
    schedule, optionally pooled); move rows with rk_gather_mean."""
    lt = np.ascontiguousarray(l_tilde, dtype=np.int32)
    p = prune_params(**params)
    return _layout_call(lib().rk_prune_layout_ex, lay, C.c_void_p(lt.ctypes.data), C.byref(p))


def rk_gather_mean(ranges: torch.Tensor, x: torch.Tensor, *, out: Optional[torch.Tensor] = None,
                   stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """y[i] = mean of rows ranges[i, 0] .. ranges[i, 1] - 1 of x (zeros for an
    empty range); arguments as rk_gather_sum."""
    return _gather(lib().rk_gather_mean, "rk_gather_mean", ranges, x, out, stream)


def rk_gather_sum(ranges: torch.Tensor, x: torch.Tensor, *, out: Optional[torch.Tensor] = None,
                  stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """y[i] = sum of rows ranges[i, 0] .. ranges[i, 1] - 1 of x (rows = first
    dimension; the rest of each row contiguous).  ranges: int32 [n, 2] on the
    device."""
    return _gather(lib().rk_gather_sum, "rk_gather_sum", ranges, x, out, stream)


def _gather(fn, name, ranges, x, out, stream):
    if ranges.dtype != torch.int32 or ranges.dim() != 2 or not ranges.is_contiguous():
        raise ValueError("ranges must be a contiguous int32 [n, 2] tensor")
    n_out = ranges.shape[0]
    width = int(np.prod(x.shape[1:])) if x.dim() > 1 else 1
    x2 = x.reshape(x.shape[0], width) if x.dim() != 2 else x
    if x2.dim() == 2 and x2.shape[0] and x2.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    if out is None:
        out = torch.empty((n_out,) + tuple(x.shape[1:]), dtype=x.dtype, device=x.device)
    y2 = out.reshape(n_out, width)
    check(fn(C.c_void_p(ranges.data_ptr()), n_out, x2.shape[0],
             C.c_void_p(x2.data_ptr()), x2.stride(0) if x2.shape[0] else width,
             C.c_void_p(y2.data_ptr()), y2.stride(0) if n_out else width, width,
             _dtype_code(x), _stream(stream)), name)
    return out
