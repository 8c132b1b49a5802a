"""ctypes mirror of include/ssd.h and the library loader.

The structures below must match the C declarations field for field (the CPU test suite
checks sizes and offsets against the header through the library's own view of them).
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssd.so")

SSD_OK = 0
SSD_ERR_NULL_POINTER = 1
SSD_ERR_BAD_SHAPE = 2
SSD_ERR_BAD_METADATA = 3
SSD_ERR_UNSUPPORTED = 4
SSD_ERR_CAPACITY = 5
SSD_ERR_WORKSPACE = 6
SSD_ERR_HIP = 7

SSD_DEVERR_CHUNK_RANGE = 1
SSD_DEVERR_SLOT_RANGE = 2
SSD_DEVERR_ACCEPTED = 4
SSD_DEVERR_CHAIN_WAIT = 8
SSD_DEVERR_DUPLICATE_SLOT = 16

SSD_F32 = 0
SSD_BF16 = 1
SSD_F16 = 2
SSD_A_SCALAR = 0
SSD_A_DIAG = 1

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_f32 = ctypes.c_float


class PrefillArgs(ctypes.Structure):
    _fields_ = [
        ("T", _i32), ("H", _i32), ("P", _i32), ("G", _i32), ("N", _i32),
        ("chunk_size", _i32), ("num_seqs", _i32), ("num_chunks", _i32),
        ("in_dtype", _i32), ("a_kind", _i32),
        ("x", _vp), ("x_stride_t", _i64),
        ("dt", _vp), ("dt_stride_t", _i64),
        ("B", _vp),
        ("C", _vp), ("bc_stride_t", _i64),
        ("y", _vp), ("y_stride_t", _i64),
        ("A", _vp), ("D", _vp), ("dt_bias", _vp),
        ("dt_softplus", _i32), ("dt_min", _f32), ("dt_max", _f32),
        ("cu_seqlens", _vp), ("cu_chunk_seqlens", _vp), ("seq_idx", _vp),
        ("last_chunk_indices", _vp),
        ("state_pool", _vp), ("slot_stride", _i64), ("num_slots", _i32),
        ("state_indices", _vp), ("has_initial_state", _vp), ("write_final_to_pool", _i32),
        ("chunk_states_out", _vp), ("device_error_flag", _vp),
        ("dA_cumsum_out", _vp), ("cb_out", _vp), ("chunk_local_states_out", _vp),
        ("profile_events", _vp), ("state_dtype", _i32),
        ("block_size", _i32), ("idx_stride", _i32), ("num_computed", _vp),
        ("block_idx_last_computed", _vp), ("block_idx_last_scheduled", _vp),
    ]


SSD_PREFILL_MAX_KERNELS = 2
SSD_NOALLOC_SCRATCH_BYTES = 256 << 20


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("B_pad", _i32), ("ntok", _i32), ("H", _i32), ("P", _i32), ("G", _i32), ("N", _i32),
        ("in_dtype", _i32), ("a_kind", _i32),
        ("x", _vp), ("dt", _vp), ("B", _vp), ("C", _vp), ("y", _vp),
        ("A", _vp), ("D", _vp), ("dt_bias", _vp),
        ("dt_softplus", _i32), ("dt_min", _f32), ("dt_max", _f32),
        ("state_pool", _vp), ("slot_stride", _i64), ("num_slots", _i32),
        ("state_indices", _vp), ("num_accepted_tokens", _vp),
        ("null_block_id", _i32), ("device_error_flag", _vp), ("profile_events", _vp),
        ("state_dtype", _i32),
        ("idx_stride", _i32), ("block_idx_last_computed", _vp),
        ("block_idx_last_scheduled", _vp),
    ]


SSD_CONV_LAYOUT_SD = 0
SSD_CONV_LAYOUT_DS = 1
SSD_CONV_MAX_KERNELS = 2


class Conv1dArgs(ctypes.Structure):
    _fields_ = [
        ("T", _i32), ("D", _i32), ("W", _i32), ("num_seqs", _i32), ("num_chunks", _i32),
        ("in_dtype", _i32),
        ("x", _vp), ("x_stride_t", _i64), ("out", _vp), ("out_stride_t", _i64),
        ("weight", _vp), ("bias", _vp), ("activation", _i32),
        ("cu_seqlens", _vp), ("cu_chunk_seqlens", _vp), ("seq_idx", _vp),
        ("conv_states", _vp), ("slot_stride", _i64), ("num_slots", _i32),
        ("state_layout", _i32), ("state_indices", _vp), ("has_initial_state", _vp),
        ("device_error_flag", _vp), ("profile_events", _vp),
    ]


class Conv1dUpdateArgs(ctypes.Structure):
    _fields_ = [
        ("B_pad", _i32), ("ntok", _i32), ("D", _i32), ("W", _i32), ("in_dtype", _i32),
        ("x", _vp), ("out", _vp), ("weight", _vp), ("bias", _vp), ("activation", _i32),
        ("conv_states", _vp), ("slot_stride", _i64), ("num_slots", _i32),
        ("state_layout", _i32), ("state_indices", _vp), ("null_block_id", _i32),
        ("device_error_flag", _vp), ("profile_events", _vp),
    ]


EXPORTS = {
    "ssd_abi_version": (ctypes.c_int, []),
    "ssd_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ssd_chunk_metadata_count": (ctypes.c_int, [_i32, _vp, _vp, _i32, _vp]),
    "ssd_build_chunk_metadata": (ctypes.c_int, [_i32, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp]),
    "ssd_prefill_workspace_size": (ctypes.c_int, [ctypes.POINTER(PrefillArgs),
                                                  ctypes.POINTER(ctypes.c_size_t)]),
    "ssd_prefill": (ctypes.c_int, [ctypes.POINTER(PrefillArgs), _vp, ctypes.c_size_t, _vp]),
    "ssd_prefill_noalloc": (ctypes.c_int, [ctypes.POINTER(PrefillArgs), _vp]),
    "ssd_prefill_kernel_count": (ctypes.c_int, [ctypes.POINTER(PrefillArgs),
                                                ctypes.POINTER(ctypes.c_int32),
                                                ctypes.POINTER(ctypes.c_char_p)]),
    "ssd_state_update": (ctypes.c_int, [ctypes.POINTER(DecodeArgs), _vp]),
    "ssd_conv1d_prefill": (ctypes.c_int, [ctypes.POINTER(Conv1dArgs), _vp]),
    "ssd_conv1d_update": (ctypes.c_int, [ctypes.POINTER(Conv1dUpdateArgs), _vp]),
    # include/ssd_probe.h (measurement aid)
    "ssd_probe_stream": (ctypes.c_int, [_vp, ctypes.c_size_t, _vp, ctypes.c_size_t, _vp,
                                        ctypes.c_int32, _vp]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libssd.so.  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m selective_state_space_mamba2_amd.build`")
        # torch ships its own HIP runtime under the same soname; loading torch first makes
        # libssd.so bind to that one instance, so torch's streams and events are valid here.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, argtypes) in EXPORTS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = argtypes
        _lib = handle
    return _lib


class SSDError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().ssd_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != SSD_OK:
        raise SSDError(fn, status)
