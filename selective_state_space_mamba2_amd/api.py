"""Python binding of the SSD C ABI: argument marshalling only.

Every function here has the name of the C entry point it calls.  Device tensors are torch
tensors (torch provides device memory and streams); every step of the scan runs in the
HIP library, and there is no other implementation to fall back on.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Sequence

import numpy as np

from . import _abi
from ._abi import DecodeArgs, PrefillArgs, check, lib

__all__ = [
    "ssd_abi_version", "ssd_status_string", "ssd_chunk_metadata_count",
    "ssd_build_chunk_metadata", "ssd_prefill_workspace_size", "ssd_prefill",
    "ssd_state_update", "prefill_args", "ssd_conv1d_prefill", "ssd_conv1d_update",
]


def ssd_abi_version() -> int:
    return lib().ssd_abi_version()


def ssd_status_string(status: int) -> str:
    return lib().ssd_status_string(status).decode()


def _i32_array(v) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(v, dtype=np.int32))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def ssd_chunk_metadata_count(cu_seqlens: Sequence[int], num_computed: Optional[Sequence[int]],
                             chunk_size: int) -> int:
    cu = _i32_array(cu_seqlens)
    nc = None if num_computed is None else _i32_array(num_computed)
    out = ctypes.c_int32(0)
    check("ssd_chunk_metadata_count",
          lib().ssd_chunk_metadata_count(len(cu) - 1, _ptr(cu), _ptr(nc), chunk_size,
                                         ctypes.byref(out)))
    return out.value


def ssd_build_chunk_metadata(cu_seqlens: Sequence[int], num_computed: Optional[Sequence[int]],
                             chunk_size: int):
    """Host chunk metadata: (cu_chunk_seqlens [C+1], seq_idx [C], last_chunk_indices [S])."""
    cu = _i32_array(cu_seqlens)
    nc = None if num_computed is None else _i32_array(num_computed)
    S = len(cu) - 1
    C = ssd_chunk_metadata_count(cu, nc, chunk_size)
    cuc = np.zeros(C + 1, dtype=np.int32)
    sidx = np.zeros(max(C, 1), dtype=np.int32)
    last = np.zeros(max(S, 1), dtype=np.int32)
    out = ctypes.c_int32(0)
    check("ssd_build_chunk_metadata",
          lib().ssd_build_chunk_metadata(S, _ptr(cu), _ptr(nc), chunk_size, C, _ptr(cuc),
                                         _ptr(sidx), _ptr(last), ctypes.byref(out)))
    return cuc, sidx[:C], last[:S]


# ----------------------------------------------------------------------------------------
# device calls (torch tensors)
# ----------------------------------------------------------------------------------------
def _dptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return _abi.SSD_BF16
    if t.dtype == torch.float32:
        return _abi.SSD_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream_ptr(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def prefill_args(x, dt, A, B, C, chunk_size: int, cu_seqlens, cu_chunk_seqlens, seq_idx,
                 last_chunk_indices, y, D=None, dt_bias=None, dt_softplus: bool = False,
                 dt_limit=(0.0, math.inf), state_pool=None, state_indices=None,
                 has_initial_state=None, write_final_to_pool: bool = False,
                 chunk_states_out=None, device_error_flag=None, dA_cumsum_out=None,
                 cb_out=None, chunk_local_states_out=None, block_size: int = 0,
                 num_computed=None, block_idx_last_computed=None,
                 block_idx_last_scheduled=None) -> PrefillArgs:
    """Fill an ssd_prefill_args from tensors (no device work).  block_size > 0 selects the
    all cache mode: state_indices is then [S, max_blocks] (row stride taken from it)."""
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    for name, t, inner in (("x", x, (P, 1)), ("y", y, (P, 1)), ("B", B, (N, 1)),
                           ("C", C, (N, 1))):
        if tuple(t.stride()[1:]) != inner:
            raise ValueError(f"{name}: each token row must be contiguous")
    if dt.stride(1) != 1 or B.stride(0) != C.stride(0):
        raise ValueError("dt rows must be contiguous and B, C must share a token stride")
    a = PrefillArgs()
    a.T, a.H, a.P, a.G, a.N = T, H, P, G, N
    a.chunk_size = int(chunk_size)
    a.num_seqs = cu_seqlens.numel() - 1
    a.num_chunks = seq_idx.numel()
    a.in_dtype = _dtype_code(x)
    a.a_kind = _abi.SSD_A_SCALAR if A.dim() == 1 else _abi.SSD_A_DIAG
    a.x, a.x_stride_t = x.data_ptr(), x.stride(0)
    a.dt, a.dt_stride_t = dt.data_ptr(), dt.stride(0)
    a.B, a.C, a.bc_stride_t = B.data_ptr(), C.data_ptr(), B.stride(0)
    a.y, a.y_stride_t = y.data_ptr(), y.stride(0)
    a.A, a.D, a.dt_bias = A.data_ptr(), _dptr(D), _dptr(dt_bias)
    a.dt_softplus = 1 if dt_softplus else 0
    a.dt_min, a.dt_max = float(dt_limit[0]), float(dt_limit[1])
    a.cu_seqlens, a.cu_chunk_seqlens = cu_seqlens.data_ptr(), cu_chunk_seqlens.data_ptr()
    a.seq_idx, a.last_chunk_indices = seq_idx.data_ptr(), last_chunk_indices.data_ptr()
    if state_pool is not None:
        a.state_pool = state_pool.data_ptr()
        a.slot_stride = state_pool.stride(0)
        a.num_slots = state_pool.shape[0]
        a.state_dtype = _dtype_code(state_pool)
    a.state_indices = _dptr(state_indices)
    a.has_initial_state = _dptr(has_initial_state)
    a.write_final_to_pool = 1 if write_final_to_pool else 0
    a.chunk_states_out = _dptr(chunk_states_out)
    a.device_error_flag = _dptr(device_error_flag)
    a.dA_cumsum_out = _dptr(dA_cumsum_out)
    a.cb_out = _dptr(cb_out)
    a.chunk_local_states_out = _dptr(chunk_local_states_out)
    a.block_size = int(block_size)
    if block_size and state_indices is not None:
        if state_indices.dim() != 2 or state_indices.stride(1) != 1:
            raise ValueError("state_indices must be [S, max_blocks] with contiguous rows")
        a.idx_stride = state_indices.stride(0)
    a.num_computed = _dptr(num_computed)
    a.block_idx_last_computed = _dptr(block_idx_last_computed)
    a.block_idx_last_scheduled = _dptr(block_idx_last_scheduled)
    return a


def ssd_prefill_workspace_size(args: PrefillArgs) -> int:
    n = ctypes.c_size_t(0)
    check("ssd_prefill_workspace_size",
          lib().ssd_prefill_workspace_size(ctypes.byref(args), ctypes.byref(n)))
    return n.value


def ssd_prefill(x, dt, A, B, C, chunk_size: int, cu_seqlens, cu_chunk_seqlens, seq_idx,
                last_chunk_indices, y=None, workspace=None, stream=None, **kw):
    """Run the chunked prefill.  Tensors follow include/ssd.h; ``y`` is allocated when not
    given, the workspace is allocated from torch when not given.  Returns y."""
    import torch
    if y is None:
        y = torch.empty_like(x)
    args = prefill_args(x, dt, A, B, C, chunk_size, cu_seqlens, cu_chunk_seqlens, seq_idx,
                        last_chunk_indices, y, **kw)
    need = ssd_prefill_workspace_size(args)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check("ssd_prefill", lib().ssd_prefill(ctypes.byref(args), ws_ptr, ws_bytes,
                                           _stream_ptr(stream)))
    return y


def decode_args(x, dt, A, B, C, y, state_pool, state_indices, num_accepted_tokens=None,
                null_block_id: int = 0, D=None, dt_bias=None, dt_softplus: bool = False,
                dt_limit=(0.0, math.inf), device_error_flag=None,
                block_idx_last_computed=None, block_idx_last_scheduled=None) -> DecodeArgs:
    """Fill an ssd_decode_args.  Passing the two block index tensors selects the all cache
    mode: state_indices is then [B_pad, max_blocks] and ntok must be 1."""
    B_pad, ntok, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    for name, t in (("x", x), ("dt", dt), ("B", B), ("C", C), ("y", y),
                    ("state_indices", state_indices)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    a = DecodeArgs()
    a.B_pad, a.ntok, a.H, a.P, a.G, a.N = B_pad, ntok, H, P, G, N
    a.in_dtype = _dtype_code(x)
    a.a_kind = _abi.SSD_A_SCALAR if A.dim() == 1 else _abi.SSD_A_DIAG
    a.x, a.dt, a.B, a.C, a.y = x.data_ptr(), dt.data_ptr(), B.data_ptr(), C.data_ptr(), y.data_ptr()
    a.A, a.D, a.dt_bias = A.data_ptr(), _dptr(D), _dptr(dt_bias)
    a.dt_softplus = 1 if dt_softplus else 0
    a.dt_min, a.dt_max = float(dt_limit[0]), float(dt_limit[1])
    a.state_pool = state_pool.data_ptr()
    a.slot_stride = state_pool.stride(0)
    a.num_slots = state_pool.shape[0]
    a.state_dtype = _dtype_code(state_pool)
    a.state_indices = state_indices.data_ptr()
    a.num_accepted_tokens = _dptr(num_accepted_tokens)
    a.null_block_id = int(null_block_id)
    a.device_error_flag = _dptr(device_error_flag)
    if block_idx_last_scheduled is not None:
        a.idx_stride = state_indices.shape[1]
        a.block_idx_last_computed = _dptr(block_idx_last_computed)
        a.block_idx_last_scheduled = _dptr(block_idx_last_scheduled)
    return a


def ssd_state_update(x, dt, A, B, C, state_pool, state_indices, y=None, stream=None, **kw):
    """Run one padded decode step in place on ``state_pool``.  Returns y."""
    import torch
    if y is None:
        y = torch.empty_like(x)
    args = decode_args(x, dt, A, B, C, y, state_pool, state_indices, **kw)
    check("ssd_state_update", lib().ssd_state_update(ctypes.byref(args), _stream_ptr(stream)))
    return y


def conv1d_args(x, weight, bias, out, cu_seqlens, cu_chunk_seqlens, seq_idx,
                activation: bool = False, conv_states=None, state_indices=None,
                has_initial_state=None, state_layout: str = "sd",
                device_error_flag=None) -> _abi.Conv1dArgs:
    """Fill an ssd_conv1d_args.  x, out [T, D] (rows contiguous); weight [D, W] fp32;
    conv_states [slots, W-1, D] ("sd") or [slots, D, W-1] ("ds") in x's dtype."""
    T, D = x.shape
    for name, t in (("x", x), ("out", out)):
        if t.stride(1) != 1:
            raise ValueError(f"{name}: each token row must be contiguous")
    if not weight.is_contiguous():
        raise ValueError("weight must be contiguous")
    a = _abi.Conv1dArgs()
    a.T, a.D, a.W = T, D, weight.shape[1]
    a.num_seqs = cu_seqlens.numel() - 1
    a.num_chunks = seq_idx.numel()
    a.in_dtype = _dtype_code(x)
    a.x, a.x_stride_t = x.data_ptr(), x.stride(0)
    a.out, a.out_stride_t = out.data_ptr(), out.stride(0)
    a.weight, a.bias = weight.data_ptr(), _dptr(bias)
    a.activation = 1 if activation else 0
    a.cu_seqlens, a.cu_chunk_seqlens = cu_seqlens.data_ptr(), cu_chunk_seqlens.data_ptr()
    a.seq_idx = seq_idx.data_ptr()
    if conv_states is not None:
        a.conv_states = conv_states.data_ptr()
        a.slot_stride = conv_states.stride(0)
        a.num_slots = conv_states.shape[0]
    a.state_layout = _abi.SSD_CONV_LAYOUT_DS if state_layout == "ds" else _abi.SSD_CONV_LAYOUT_SD
    a.state_indices = _dptr(state_indices)
    a.has_initial_state = _dptr(has_initial_state)
    a.device_error_flag = _dptr(device_error_flag)
    return a


def ssd_conv1d_prefill(x, weight, bias, cu_seqlens, cu_chunk_seqlens, seq_idx, out=None,
                       stream=None, **kw):
    """Run the varlen causal conv1d (states updated in place when a pool is given).
    Returns out."""
    import torch
    if out is None:
        out = torch.empty_like(x)
    args = conv1d_args(x, weight, bias, out, cu_seqlens, cu_chunk_seqlens, seq_idx, **kw)
    check("ssd_conv1d_prefill", lib().ssd_conv1d_prefill(ctypes.byref(args),
                                                         _stream_ptr(stream)))
    return out


def conv1d_update_args(x, weight, bias, out, conv_states, state_indices,
                       activation: bool = False, null_block_id: int = 0,
                       state_layout: str = "sd", device_error_flag=None) -> _abi.Conv1dUpdateArgs:
    """Fill an ssd_conv1d_update_args.  x, out [B_pad, ntok, D] contiguous."""
    B_pad, ntok, D = x.shape
    for name, t in (("x", x), ("out", out), ("weight", weight),
                    ("state_indices", state_indices)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    a = _abi.Conv1dUpdateArgs()
    a.B_pad, a.ntok, a.D, a.W = B_pad, ntok, D, weight.shape[1]
    a.in_dtype = _dtype_code(x)
    a.x, a.out, a.weight, a.bias = x.data_ptr(), out.data_ptr(), weight.data_ptr(), _dptr(bias)
    a.activation = 1 if activation else 0
    a.conv_states = conv_states.data_ptr()
    a.slot_stride = conv_states.stride(0)
    a.num_slots = conv_states.shape[0]
    a.state_layout = _abi.SSD_CONV_LAYOUT_DS if state_layout == "ds" else _abi.SSD_CONV_LAYOUT_SD
    a.state_indices = state_indices.data_ptr()
    a.null_block_id = int(null_block_id)
    a.device_error_flag = _dptr(device_error_flag)
    return a


def ssd_conv1d_update(x, weight, bias, conv_states, state_indices, out=None, stream=None,
                      **kw):
    """One decode step of the conv, in place on ``conv_states``.  Returns out."""
    import torch
    if out is None:
        out = torch.empty_like(x)
    args = conv1d_update_args(x, weight, bias, out, conv_states, state_indices, **kw)
    check("ssd_conv1d_update", lib().ssd_conv1d_update(ctypes.byref(args), _stream_ptr(stream)))
    return out
