"""ctypes declarations of the C ABI in include/rk.h (argument marshalling only).

The library is loaded from this package directory (librk.so, built by
masked_attention_amd/build.py).  Loading fails loudly when it is missing:
there is no fallback implementation.
"""

from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librk.so")

RK_OK = 0
RK_ERR_INVALID_ARG = 1
RK_ERR_SEGMENT_ORDER = 2
RK_ERR_UNSORTED_TIME = 3
RK_ERR_UNSUPPORTED = 4
RK_ERR_WORKSPACE_TOO_SMALL = 5
RK_ERR_HIP = 6

RK_F32 = 0
RK_BF16 = 1

RK_SEG_PROFILE, RK_SEG_HISTORY, RK_SEG_REALTIME, RK_SEG_CANDIDATE = 0, 1, 2, 3
RK_TILE_EMPTY, RK_TILE_PARTIAL, RK_TILE_FULL = 0, 1, 2
RK_TILE_Q, RK_TILE_K = 128, 64
RK_STATIC_BIDIRECTIONAL = 0x1
RK_QUERY_CANDIDATES_ONLY = 0x2
RK_PLAN_BACKWARD = 0x4
RK_ATTN_REFERENCE_KERNEL = 0x1
RK_ATTN_K_PREROTATED = 0x2
RK_ABI_VERSION = 4
RK_SPLIT_SLOTS = 768  # extra work-list slots of a candidates-only plan
RK_PRUNE_LINEAR = 0
RK_PRUNE_EXP = 1


class rk_batch(C.Structure):
    _fields_ = [
        ("struct_size", C.c_uint32),
        ("num_requests", C.c_int32),
        ("total_tokens", C.c_int32),
        ("req_offsets_host", C.c_void_p),
        ("req_offsets_dev", C.c_void_p),
        ("seg_kind_dev", C.c_void_p),
        ("timestamps_dev", C.c_void_p),
        ("anchors_dev", C.c_void_p),
    ]


class rk_mask_params(C.Structure):
    _fields_ = [
        ("struct_size", C.c_uint32),
        ("flags", C.c_uint32),
        ("delay", C.c_int64),
        ("window", C.c_int32),
        ("global_tail", C.c_int32),
    ]


class rk_rope_params(C.Structure):
    _fields_ = [
        ("struct_size", C.c_uint32),
        ("kinds", C.c_uint32),
        ("phi_min", C.c_double),
        ("dt_max", C.c_double),
        ("base", C.c_double),
    ]


class rk_qk_norm_params(C.Structure):
    _fields_ = [
        ("struct_size", C.c_uint32),
        ("eps", C.c_float),
        ("gamma_q", C.c_void_p),
        ("gamma_k", C.c_void_p),
    ]


class rk_plan_info(C.Structure):
    _fields_ = [
        ("struct_size", C.c_uint32),
        ("num_requests", C.c_int32),
        ("total_tokens", C.c_int32),
        ("num_heads", C.c_int32),
        ("num_qtiles", C.c_int64),
        ("num_tiles", C.c_int64),
        ("num_sched_slots", C.c_int64),
        ("workspace", C.c_void_p),
        ("off_tile_class", C.c_size_t),
        ("off_tile_count", C.c_size_t),
        ("off_qtile_ptr", C.c_size_t),
        ("off_ktile_idx", C.c_size_t),
        ("off_row_desc", C.c_size_t),
        ("off_sched", C.c_size_t),
        ("num_work_slots", C.c_int64),
        ("off_work", C.c_size_t),
        ("off_splits", C.c_size_t),
        ("num_kblocks", C.c_int64),
        ("num_ksched_slots", C.c_int64),
        ("off_kt_ptr", C.c_size_t),
        ("off_qtile_word", C.c_size_t),
        ("off_ksched", C.c_size_t),
    ]


class rk_plan_totals(C.Structure):
    _fields_ = [
        ("struct_size", C.c_uint32),
        ("device_errors", C.c_uint32),
        ("visible_pairs", C.c_int64),
        ("full_tiles", C.c_int64),
        ("partial_tiles", C.c_int64),
        ("empty_tiles", C.c_int64),
        ("work_entries", C.c_int32),
        ("split_items", C.c_int32),
    ]


class rk_attn_args(C.Structure):
    _fields_ = [
        ("struct_size", C.c_uint32),
        ("flags", C.c_uint32),
        ("dtype", C.c_int),
        ("num_heads", C.c_int32),
        ("d_head", C.c_int32),
        ("reserved", C.c_int32),
        ("q", C.c_void_p),
        ("k", C.c_void_p),
        ("v", C.c_void_p),
        ("o", C.c_void_p),
        ("lse", C.c_void_p),
        ("q_stride_tok", C.c_int64), ("q_stride_head", C.c_int64),
        ("k_stride_tok", C.c_int64), ("k_stride_head", C.c_int64),
        ("v_stride_tok", C.c_int64), ("v_stride_head", C.c_int64),
        ("o_stride_tok", C.c_int64), ("o_stride_head", C.c_int64),
        ("scale", C.c_float),
        ("reserved2", C.c_float),
        ("rope", C.c_void_p),
        ("workspace", C.c_void_p),
        ("workspace_bytes", C.c_size_t),
        ("qk_norm", C.c_void_p),
    ]


class rk_attn_bwd_args(C.Structure):
    _fields_ = [
        ("struct_size", C.c_uint32),
        ("flags", C.c_uint32),
        ("dtype", C.c_int),
        ("num_heads", C.c_int32),
        ("d_head", C.c_int32),
        ("reserved", C.c_int32),
        ("q", C.c_void_p),
        ("k", C.c_void_p),
        ("v", C.c_void_p),
        ("o", C.c_void_p),
        ("d_o", C.c_void_p),
        ("lse", C.c_void_p),
        ("dq", C.c_void_p),
        ("dk", C.c_void_p),
        ("dv", C.c_void_p),
        ("q_stride_tok", C.c_int64), ("q_stride_head", C.c_int64),
        ("k_stride_tok", C.c_int64), ("k_stride_head", C.c_int64),
        ("v_stride_tok", C.c_int64), ("v_stride_head", C.c_int64),
        ("o_stride_tok", C.c_int64), ("o_stride_head", C.c_int64),
        ("do_stride_tok", C.c_int64), ("do_stride_head", C.c_int64),
        ("dq_stride_tok", C.c_int64), ("dq_stride_head", C.c_int64),
        ("dk_stride_tok", C.c_int64), ("dk_stride_head", C.c_int64),
        ("dv_stride_tok", C.c_int64), ("dv_stride_head", C.c_int64),
        ("scale", C.c_float),
        ("reserved2", C.c_float),
        ("rope", C.c_void_p),
        ("workspace", C.c_void_p),
        ("workspace_bytes", C.c_size_t),
        ("qk_norm", C.c_void_p),
        ("dgamma_q", C.c_void_p),
        ("dgamma_k", C.c_void_p),
    ]


class rk_pointwise_args(C.Structure):
    _fields_ = [
        ("struct_size", C.c_uint32),
        ("flags", C.c_uint32),
        ("dtype", C.c_int),
        ("num_heads", C.c_int32),
        ("d_head", C.c_int32),
        ("num_pos_buckets", C.c_int32),
        ("q", C.c_void_p),
        ("k", C.c_void_p),
        ("v", C.c_void_p),
        ("o", C.c_void_p),
        ("q_stride_tok", C.c_int64), ("q_stride_head", C.c_int64),
        ("k_stride_tok", C.c_int64), ("k_stride_head", C.c_int64),
        ("v_stride_tok", C.c_int64), ("v_stride_head", C.c_int64),
        ("o_stride_tok", C.c_int64), ("o_stride_head", C.c_int64),
        ("scale", C.c_float),
        ("num_time_buckets", C.c_int32),
        ("pos_bias", C.c_void_p),
        ("time_bias", C.c_void_p),
    ]


class rk_host_layout(C.Structure):
    _fields_ = [
        ("struct_size", C.c_uint32),
        ("num_requests", C.c_int32),
        ("total_tokens", C.c_int32),
        ("reserved", C.c_int32),
        ("req_offsets", C.c_void_p),
        ("seg_kind", C.c_void_p),
        ("timestamps", C.c_void_p),
    ]


class rk_layout_out(C.Structure):
    _fields_ = [
        ("struct_size", C.c_uint32),
        ("capacity", C.c_int32),
        ("total_tokens", C.c_int32),
        ("reserved", C.c_int32),
        ("req_offsets", C.c_void_p),
        ("seg_kind", C.c_void_p),
        ("timestamps", C.c_void_p),
        ("ranges", C.c_void_p),
    ]


class rk_prune_params(C.Structure):
    _fields_ = [
        ("struct_size", C.c_uint32),
        ("schedule", C.c_int32),
        ("n_min", C.c_int32),
        ("layer", C.c_int32),
        ("num_layers", C.c_int32),
        ("pool", C.c_int32),
        ("decay", C.c_double),
    ]


STRUCTS = {
    "rk_batch": rk_batch,
    "rk_mask_params": rk_mask_params,
    "rk_rope_params": rk_rope_params,
    "rk_qk_norm_params": rk_qk_norm_params,
    "rk_plan_info": rk_plan_info,
    "rk_plan_totals": rk_plan_totals,
    "rk_attn_args": rk_attn_args,
    "rk_attn_bwd_args": rk_attn_bwd_args,
    "rk_pointwise_args": rk_pointwise_args,
    "rk_host_layout": rk_host_layout,
    "rk_layout_out": rk_layout_out,
    "rk_prune_params": rk_prune_params,
}

# (name, restype, argtypes) of every exported entry point
FUNCTIONS = [
    ("rk_status_string", C.c_char_p, [C.c_int]),
    ("rk_abi_version", C.c_int32, []),
    ("rk_plan_workspace_size", C.c_int, [C.POINTER(rk_batch), C.c_int32, C.POINTER(C.c_size_t)]),
    ("rk_mask_plan", C.c_int, [C.POINTER(rk_batch), C.POINTER(rk_mask_params), C.c_int32,
                               C.c_void_p, C.c_size_t, C.POINTER(C.c_void_p), C.c_void_p]),
    ("rk_plan_get_info", C.c_int, [C.c_void_p, C.POINTER(rk_plan_info)]),
    ("rk_plan_stats", C.c_int, [C.c_void_p, C.POINTER(rk_plan_totals), C.c_void_p]),
    ("rk_plan_destroy", None, [C.c_void_p]),
    ("rk_time_rope", C.c_int, [C.POINTER(rk_batch), C.POINTER(rk_rope_params), C.c_void_p,
                               C.c_void_p, C.c_int, C.c_int32, C.c_int32, C.c_int64, C.c_int64,
                               C.c_int64, C.c_int64, C.c_void_p]),
    ("rk_qk_norm_rope", C.c_int, [C.POINTER(rk_batch), C.POINTER(rk_rope_params), C.c_float,
                                  C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_int32,
                                  C.c_int32, C.c_int64, C.c_int64, C.c_int64, C.c_int64,
                                  C.c_void_p]),
    ("rk_attn_workspace_size", C.c_int, [C.c_void_p, C.POINTER(rk_attn_args),
                                         C.POINTER(C.c_size_t)]),
    ("rk_masked_attn_fwd", C.c_int, [C.c_void_p, C.POINTER(rk_attn_args), C.c_void_p]),
    ("rk_masked_attn_fwd_noalloc", C.c_int, [C.c_void_p, C.POINTER(rk_attn_args), C.c_void_p]),
    ("rk_attn_bwd_workspace_size", C.c_int, [C.c_void_p, C.POINTER(rk_attn_bwd_args),
                                             C.POINTER(C.c_size_t)]),
    ("rk_masked_attn_bwd", C.c_int, [C.c_void_p, C.POINTER(rk_attn_bwd_args), C.c_void_p]),
    ("rk_pointwise_attn_fwd", C.c_int, [C.c_void_p, C.POINTER(rk_pointwise_args), C.c_void_p]),
    ("rk_compress_layout", C.c_int, [C.POINTER(rk_host_layout), C.c_int32, C.c_int32,
                                     C.POINTER(rk_layout_out)]),
    ("rk_pruned_history_length", C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                           C.POINTER(C.c_int32)]),
    ("rk_prune_layout", C.c_int, [C.POINTER(rk_host_layout), C.c_void_p, C.c_int32, C.c_int32,
                                  C.c_int32, C.POINTER(rk_layout_out)]),
    ("rk_gather_sum", C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_int64,
                                C.c_void_p, C.c_int64, C.c_int32, C.c_int, C.c_void_p]),
    ("rk_pruned_history_length_ex", C.c_int, [C.c_int32, C.POINTER(rk_prune_params),
                                              C.POINTER(C.c_int32)]),
    ("rk_prune_layout_ex", C.c_int, [C.POINTER(rk_host_layout), C.c_void_p,
                                     C.POINTER(rk_prune_params), C.POINTER(rk_layout_out)]),
    ("rk_gather_mean", C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_int64,
                                 C.c_void_p, C.c_int64, C.c_int32, C.c_int, C.c_void_p]),
]

_lib = None


def lib() -> C.CDLL:
    """Load librk.so (once) and declare its entry points."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (python -m masked_attention_amd.build); "
                "there is no non-HIP fallback")
        L = C.CDLL(LIB_PATH)
        for name, res, args in FUNCTIONS:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class RkError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib().rk_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


def check(status: int, where: str) -> None:
    if status != RK_OK:
        raise RkError(status, where)


def sized(cls, **kw):
    s = cls(**kw)
    s.struct_size = C.sizeof(cls)
    return s
