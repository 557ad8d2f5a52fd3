"""ctypes view of include/hstu.h and the loader of libhstu.so.

Argument marshalling only.  Loading fails loudly when the library has not
been built: there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhstu.so")

HSTU_OK = 0
HSTU_ERR_ARG = -1
HSTU_ERR_UNSUPPORTED = -2
HSTU_ERR_WORKSPACE = -3
HSTU_ERR_DEVICE = -4

HSTU_F32 = 0
HSTU_BF16 = 1
HSTU_ACT_SILU = 0
HSTU_ACT_IDENTITY = 1

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("B", _i32), ("H", _i32), ("d_qk", _i32), ("d_v", _i32),
        ("max_seq_len", _i32),
        ("num_rows", _i64),
        ("seq_offsets", _vp), ("seq_lengths", _vp), ("num_candidates", _vp),
        ("dtype", _i32), ("act", _i32),
        ("q", _vp), ("q_stride", _i64),
        ("k", _vp), ("k_stride", _i64),
        ("v", _vp), ("v_stride", _i64),
        ("timestamps", _vp),
        ("rab_pos", _vp), ("num_pos_buckets", _i32), ("rab_pos_head_stride", _i32),
        ("rab_time", _vp), ("num_time_buckets", _i32), ("rab_time_head_stride", _i32),
        ("alpha", _f32),
        ("o", _vp), ("o_stride", _i64),
        ("u", _vp), ("u_stride", _i64),
        ("y", _vp), ("y_stride", _i64),
        ("ln_eps", _f32),
        ("ev_core_begin", _vp), ("ev_core_end", _vp),
        ("ev_epi_begin", _vp), ("ev_epi_end", _vp),
    ]


class MfalconArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("attn", AttnArgs),
        ("w", _vp),
        ("scores", _vp),
        ("score_stride", _i32),
        ("candidates_only", _i32),
    ]


class MfalconCachedArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("B", _i32), ("H", _i32), ("d", _i32),
        ("max_hist_len", _i32), ("max_cands", _i32),
        ("hist_offsets", _vp), ("num_hist_rows", _i64),
        ("k_hist", _vp), ("k_hist_stride", _i64),
        ("v_hist", _vp), ("v_hist_stride", _i64),
        ("ts_hist", _vp),
        ("cand_offsets", _vp), ("num_cand_rows", _i64),
        ("q", _vp), ("q_stride", _i64),
        ("k", _vp), ("k_stride", _i64),
        ("v", _vp), ("v_stride", _i64),
        ("u", _vp), ("u_stride", _i64),
        ("ts_cand", _vp),
        ("rab_pos", _vp), ("num_pos_buckets", _i32), ("rab_pos_head_stride", _i32),
        ("rab_time", _vp), ("num_time_buckets", _i32), ("rab_time_head_stride", _i32),
        ("alpha", _f32),
        ("ln_eps", _f32),
        ("w", _vp),
        ("scores", _vp),
        ("score_stride", _i32),
        ("o", _vp), ("o_stride", _i64),
        ("ev_core_begin", _vp), ("ev_core_end", _vp),
    ]


class AttnBwdArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("attn", AttnArgs),
        ("dy", _vp), ("dy_stride", _i64),
        ("dout", _vp), ("dout_stride", _i64),
        ("dq", _vp), ("dq_stride", _i64),
        ("dk", _vp), ("dk_stride", _i64),
        ("dv", _vp), ("dv_stride", _i64),
        ("du", _vp), ("du_stride", _i64),
        ("drab_pos", _vp), ("drab_time", _vp),
        ("ev_dq_begin", _vp), ("ev_dq_end", _vp),
        ("ev_dkv_begin", _vp), ("ev_dkv_end", _vp),
    ]


class LayerArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("B", _i32), ("H", _i32), ("d", _i32), ("D", _i32),
        ("max_seq_len", _i32),
        ("num_rows", _i64),
        ("seq_offsets", _vp), ("num_candidates", _vp),
        ("x", _vp), ("w1", _vp), ("b1", _vp), ("w2", _vp), ("b2", _vp),
        ("timestamps", _vp),
        ("rab_pos", _vp), ("num_pos_buckets", _i32),
        ("rab_time", _vp), ("num_time_buckets", _i32),
        ("alpha", _f32), ("ln_eps", _f32),
        ("x_out", _vp),
    ]


class MfalconLayerArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("layer", LayerArgs),
        ("w", _vp),
        ("scores", _vp),
        ("score_stride", _i32),
        ("candidates_only", _i32),
    ]


class LayerBwdArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("layer", LayerArgs),
        ("dx_out", _vp), ("dx", _vp),
        ("dw1", _vp), ("db1", _vp), ("dw2", _vp), ("db2", _vp),
        ("drab_pos", _vp), ("drab_time", _vp),
    ]


SL_MAX_TENSORS = 8


class SlArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("B", _i32),
        ("num_rows", _i64),
        ("seq_offsets", _vp),
        ("cap", _i32),
        ("caps", _vp),
        ("seed", ctypes.c_uint64),
        ("step", ctypes.c_uint64),
        ("out_offsets", _vp),
        ("out_index", _vp),
        ("num_tensors", _i32),
        ("src", _vp * SL_MAX_TENSORS),
        ("src_stride", _i64 * SL_MAX_TENSORS),
        ("dst", _vp * SL_MAX_TENSORS),
        ("dst_stride", _i64 * SL_MAX_TENSORS),
        ("row_bytes", _i32 * SL_MAX_TENSORS),
    ]


# every symbol include/hstu.h declares
EXPORTS = [
    "hstu_abi_version", "hstu_status_string", "hstu_last_error",
    "hstu_attn_workspace_bytes", "hstu_attn_fwd",
    "hstu_attn_fwd_noalloc", "hstu_attn_noalloc_scratch_bytes",
    "hstu_mfalcon_workspace_bytes", "mfalcon_score",
    "hstu_mfalcon_cached_workspace_bytes", "mfalcon_score_cached",
    "hstu_layer_workspace_bytes", "hstu_layer_fwd",
    "hstu_mfalcon_layer_workspace_bytes", "mfalcon_layer_score",
    "hstu_attn_bwd_workspace_bytes", "hstu_attn_bwd",
    "hstu_layer_bwd_workspace_bytes", "hstu_layer_bwd",
    "hstu_layer_saved_bytes", "hstu_layer_fwd_saved", "hstu_layer_bwd_saved",
    "hstu_layer_bwd_saved_workspace_bytes",
    "hstu_stochastic_length",
    "hstu_attn_schedule",
    "hstu_validate_offsets",
]

_LIB = None


class HstuError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"hstu status {status}: {msg}")
        self.status = status


def load(path: str = LIB_PATH):
    """Load libhstu.so (cached).  Raises if it is missing: build it first."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python -m hstu_sequential_transducer_causal_amd.build)")
    lib = ctypes.CDLL(path)
    lib.hstu_abi_version.restype = ctypes.c_int
    lib.hstu_status_string.restype = ctypes.c_char_p
    lib.hstu_status_string.argtypes = [_i32]
    lib.hstu_last_error.restype = ctypes.c_char_p
    lib.hstu_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.hstu_attn_workspace_bytes.argtypes = [ctypes.POINTER(AttnArgs)]
    lib.hstu_attn_fwd.restype = _i32
    lib.hstu_attn_fwd.argtypes = [ctypes.POINTER(AttnArgs), _vp, ctypes.c_size_t, _vp]
    lib.hstu_attn_fwd_noalloc.restype = _i32
    lib.hstu_attn_fwd_noalloc.argtypes = [ctypes.POINTER(AttnArgs), _vp]
    lib.hstu_attn_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.hstu_attn_noalloc_scratch_bytes.argtypes = []
    lib.hstu_mfalcon_workspace_bytes.restype = ctypes.c_size_t
    lib.hstu_mfalcon_workspace_bytes.argtypes = [ctypes.POINTER(MfalconArgs)]
    lib.mfalcon_score.restype = _i32
    lib.mfalcon_score.argtypes = [ctypes.POINTER(MfalconArgs), _vp, ctypes.c_size_t, _vp]
    lib.hstu_mfalcon_cached_workspace_bytes.restype = ctypes.c_size_t
    lib.hstu_mfalcon_cached_workspace_bytes.argtypes = [ctypes.POINTER(MfalconCachedArgs)]
    lib.mfalcon_score_cached.restype = _i32
    lib.mfalcon_score_cached.argtypes = [ctypes.POINTER(MfalconCachedArgs), _vp, ctypes.c_size_t, _vp]
    lib.hstu_layer_workspace_bytes.restype = ctypes.c_size_t
    lib.hstu_layer_workspace_bytes.argtypes = [ctypes.POINTER(LayerArgs)]
    lib.hstu_layer_fwd.restype = _i32
    lib.hstu_layer_fwd.argtypes = [ctypes.POINTER(LayerArgs), _vp, ctypes.c_size_t, _vp]
    lib.hstu_mfalcon_layer_workspace_bytes.restype = ctypes.c_size_t
    lib.hstu_mfalcon_layer_workspace_bytes.argtypes = [ctypes.POINTER(MfalconLayerArgs)]
    lib.mfalcon_layer_score.restype = _i32
    lib.mfalcon_layer_score.argtypes = [ctypes.POINTER(MfalconLayerArgs), _vp, ctypes.c_size_t, _vp]
    lib.hstu_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.hstu_attn_bwd_workspace_bytes.argtypes = [ctypes.POINTER(AttnBwdArgs)]
    lib.hstu_attn_bwd.restype = _i32
    lib.hstu_attn_bwd.argtypes = [ctypes.POINTER(AttnBwdArgs), _vp, ctypes.c_size_t, _vp]
    lib.hstu_layer_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.hstu_layer_bwd_workspace_bytes.argtypes = [ctypes.POINTER(LayerBwdArgs)]
    lib.hstu_layer_bwd.restype = _i32
    lib.hstu_layer_bwd.argtypes = [ctypes.POINTER(LayerBwdArgs), _vp, ctypes.c_size_t, _vp]
    lib.hstu_layer_saved_bytes.restype = ctypes.c_size_t
    lib.hstu_layer_saved_bytes.argtypes = [ctypes.POINTER(LayerArgs)]
    lib.hstu_layer_fwd_saved.restype = _i32
    lib.hstu_layer_fwd_saved.argtypes = [ctypes.POINTER(LayerArgs), _vp, ctypes.c_size_t, _vp, ctypes.c_size_t, _vp]
    lib.hstu_layer_bwd_saved_workspace_bytes.restype = ctypes.c_size_t
    lib.hstu_layer_bwd_saved_workspace_bytes.argtypes = [ctypes.POINTER(LayerBwdArgs)]
    lib.hstu_layer_bwd_saved.restype = _i32
    lib.hstu_layer_bwd_saved.argtypes = [ctypes.POINTER(LayerBwdArgs), _vp, ctypes.c_size_t, _vp, ctypes.c_size_t,
                                         _vp]
    lib.hstu_stochastic_length.restype = _i32
    lib.hstu_stochastic_length.argtypes = [ctypes.POINTER(SlArgs), _vp]
    lib.hstu_attn_schedule.restype = _i32
    lib.hstu_attn_schedule.argtypes = [ctypes.POINTER(AttnArgs), _vp, ctypes.c_size_t,
                                       ctypes.POINTER(_i32), _i64, ctypes.POINTER(_i64),
                                       ctypes.POINTER(_i32), ctypes.POINTER(_i32), _vp]
    lib.hstu_validate_offsets.restype = _i32
    lib.hstu_validate_offsets.argtypes = [ctypes.POINTER(AttnArgs), _vp]
    _LIB = lib
    return lib


def check(status: int) -> None:
    if status != HSTU_OK:
        lib = load()
        raise HstuError(status, lib.hstu_last_error().decode(errors="replace")
                        or lib.hstu_status_string(status).decode())
