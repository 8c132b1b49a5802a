"""Python binding of the SSD C ABI: argument marshalling only.

Every function here has the name of the C entry point it calls.  Device tensors are torch
tensors (torch provides device memory and streams); every step of the scan runs in the
HIP library, and there is no other implementation to fall back on.

Before anything is handed to the library, every tensor is checked for what the C ABI
assumes of the memory behind its pointer: on the GPU of ``x`` (a host pointer given to a
kernel would fault the GPU), the dtype the header declares (int32 metadata and indices,
fp32 parameters, token tensors in x's dtype), contiguous where the ABI takes no stride,
and the element count the sizes imply.  A violation raises ValueError and launches
nothing.

Device-side errors (an index out of range, inconsistent chunk metadata) are OR-ed into
an int32 error word.  A call given no ``device_error_flag`` uses a persistent error word
of its GPU, so such errors are never lost: ``ssd_device_errors`` reads it (and
synchronises the device), ``check_device_errors`` raises when it is set.
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
    "ssd_device_errors", "check_device_errors", "device_error_names", "ssd_prefill_noalloc",
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
    if t.dtype == torch.float16:
        return _abi.SSD_F16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream_ptr(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


_DEVERR_NAMES = [(_abi.SSD_DEVERR_CHUNK_RANGE, "CHUNK_RANGE"),
                 (_abi.SSD_DEVERR_SLOT_RANGE, "SLOT_RANGE"),
                 (_abi.SSD_DEVERR_ACCEPTED, "ACCEPTED"),
                 (_abi.SSD_DEVERR_CHAIN_WAIT, "CHAIN_WAIT"),
                 (_abi.SSD_DEVERR_DUPLICATE_SLOT, "DUPLICATE_SLOT")]
_ERROR_WORDS = {}


def _error_word(device):
    """The persistent int32 error word of a GPU (allocated zeroed on first use)."""
    import torch
    idx = torch.device(device).index
    idx = torch.cuda.current_device() if idx is None else idx
    w = _ERROR_WORDS.get(idx)
    if w is None:
        w = torch.zeros(1, dtype=torch.int32, device=f"cuda:{idx}")
        _ERROR_WORDS[idx] = w
    return w


def device_error_names(bits: int):
    """Names of the SSD_DEVERR_* bits set in ``bits``."""
    return [n for b, n in _DEVERR_NAMES if bits & b]


def ssd_device_errors(device=None, clear: bool = True) -> int:
    """SSD_DEVERR_* bits raised on ``device`` (default: the current GPU) by calls that were
    given no device_error_flag, since the last clear.  Synchronises the device."""
    import torch
    w = _error_word("cuda" if device is None else device)
    torch.cuda.synchronize(w.device)
    bits = int(w.item())
    if clear and bits:
        w.zero_()
    return bits


def check_device_errors(device=None) -> None:
    """Raise RuntimeError if a call without its own device_error_flag raised a device-side
    error on ``device`` (the error word is cleared)."""
    bits = ssd_device_errors(device)
    if bits:
        raise RuntimeError(f"SSD device error bits 0x{bits:x}: {', '.join(device_error_names(bits))}")


class _Checker:
    """Argument checks of one call: everything on ``device``, the declared dtypes, the
    memory layout the ABI assumes and the element counts the sizes imply."""

    def __init__(self, fn: str, ref):
        self.fn = fn
        self.device = ref.device
        self.refs = []      # every tensor the argument struct will point into

    def keep(self, a):
        """Attach the checked tensors to the argument struct ``a``: the struct holds raw
        device addresses, so the tensors behind them must live as long as it does."""
        a._tensors = tuple(self.refs)
        return a

    def fail(self, msg):
        raise ValueError(f"{self.fn}: {msg}")

    def t(self, name, t, dtypes=None, numel=None, contiguous=False, min_numel=None):
        import torch
        if t is None:
            return
        if not isinstance(t, torch.Tensor):
            self.fail(f"{name} must be a torch tensor")
        if dtypes is not None and t.dtype not in dtypes:
            self.fail(f"{name} has dtype {t.dtype}, expected {' or '.join(map(str, dtypes))}")
        if contiguous and not t.is_contiguous():
            self.fail(f"{name} must be contiguous")
        if numel is not None and t.numel() != numel:
            self.fail(f"{name} has {t.numel()} elements, expected {numel}")
        if min_numel is not None and t.numel() < min_numel:
            self.fail(f"{name} has {t.numel()} elements, expected at least {min_numel}")
        if t.device != self.device:
            self.fail(f"{name} is on {t.device}, expected {self.device} (the device of the "
                      f"token tensors)")
        self.refs.append(t)

    def i32(self, name, t, numel=None, min_numel=None):
        import torch
        self.t(name, t, (torch.int32,), numel=numel, contiguous=True, min_numel=min_numel)

    def f32(self, name, t, numel=None):
        import torch
        self.t(name, t, (torch.float32,), numel=numel, contiguous=True)

    def gpu(self, name, t):
        if not t.is_cuda:
            self.fail(f"{name} must be a GPU tensor (got {t.device})")


def _float_dtypes():
    import torch
    return (torch.bfloat16, torch.float32)


def _pool_dtypes():
    import torch
    return (torch.bfloat16, torch.float32, torch.float16)


def _flag_for(ck: _Checker, device_error_flag):
    """The caller's error flag, or the GPU's persistent error word."""
    return _error_word(ck.device) if device_error_flag is None else device_error_flag


def prefill_args(x, dt, A, B, C, chunk_size: int, cu_seqlens, cu_chunk_seqlens, seq_idx,
                 last_chunk_indices, y, D=None, dt_bias=None, dt_softplus: bool = False,
                 dt_limit=(0.0, math.inf), state_pool=None, state_indices=None,
                 has_initial_state=None, write_final_to_pool: bool = False,
                 chunk_states_out=None, device_error_flag=None, dA_cumsum_out=None,
                 cb_out=None, chunk_local_states_out=None, block_size: int = 0,
                 num_computed=None, block_idx_last_computed=None,
                 block_idx_last_scheduled=None) -> PrefillArgs:
    """Fill an ssd_prefill_args from tensors (no device work).  block_size > 0 selects the
    all cache mode: state_indices is then [S, max_blocks] (row stride taken from it).  The
    returned struct holds the tensors it points into (``_tensors``), so they live as long
    as it does; the same holds for the other argument builders below."""
    import torch
    ck = _Checker("ssd_prefill", x)
    if x.dim() != 3 or B.dim() != 3 or C.dim() != 3 or dt.dim() != 2 or y.dim() != 3:
        ck.fail("x, y must be [T, H, P], dt [T, H], B and C [T, G, N]")
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    ck.t("x", x, _float_dtypes())
    for name, t in (("dt", dt), ("B", B), ("C", C), ("y", y)):
        ck.t(name, t, (x.dtype,))
    if tuple(dt.shape) != (T, H) or tuple(y.shape) != (T, H, P) or tuple(C.shape) != (T, G, N) \
            or B.shape[0] != T:
        ck.fail("dt, B, C and y must match x's tokens and heads")
    for name, t, inner in (("x", x, (P, 1)), ("y", y, (P, 1)), ("B", B, (N, 1)),
                           ("C", C, (N, 1))):
        if tuple(t.stride()[1:]) != inner:
            raise ValueError(f"{name}: each token row must be contiguous")
    if dt.stride(1) != 1 or B.stride(0) != C.stride(0):
        raise ValueError("dt rows must be contiguous and B, C must share a token stride")
    S = cu_seqlens.numel() - 1
    Cn = seq_idx.numel()
    diag = A.dim() == 2
    ck.f32("A", A, numel=H * N if diag else H)
    ck.f32("D", D, numel=H)
    ck.f32("dt_bias", dt_bias, numel=H)
    ck.i32("cu_seqlens", cu_seqlens)
    ck.i32("cu_chunk_seqlens", cu_chunk_seqlens, numel=Cn + 1)
    ck.i32("seq_idx", seq_idx)
    ck.i32("last_chunk_indices", last_chunk_indices, numel=S)
    if state_pool is not None:
        ck.t("state_pool", state_pool, _pool_dtypes())
        if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, P, N) or \
                tuple(state_pool.stride()[1:]) != (P * N, N, 1):
            ck.fail("state_pool must be [slots, H, P, N] with contiguous slots")
    if state_indices is not None:
        ck.t("state_indices", state_indices, (torch.int32,))
        if state_indices.stride(-1) != 1 or state_indices.dim() > 2 or \
                (not block_size and state_indices.numel() != S) or \
                (block_size and (state_indices.dim() != 2 or state_indices.shape[0] != S)):
            ck.fail("state_indices must be [S] (or [S, max_blocks] in the all cache mode) "
                    "with contiguous rows")
    ck.i32("has_initial_state", has_initial_state, numel=S)
    ck.f32("chunk_states_out", chunk_states_out, numel=Cn * H * P * N)
    ck.f32("dA_cumsum_out", dA_cumsum_out, numel=H * T)
    ck.f32("cb_out", cb_out, numel=Cn * G * chunk_size * chunk_size)
    ck.f32("chunk_local_states_out", chunk_local_states_out, numel=Cn * H * P * N)
    ck.i32("num_computed", num_computed, numel=S)
    ck.i32("block_idx_last_computed", block_idx_last_computed, numel=S)
    ck.i32("block_idx_last_scheduled", block_idx_last_scheduled, numel=S)
    ck.i32("device_error_flag", device_error_flag, min_numel=1)
    ck.gpu("x", x)     # every other tensor is on x's device
    device_error_flag = _flag_for(ck, device_error_flag)
    a = PrefillArgs()
    a.T, a.H, a.P, a.G, a.N = T, H, P, G, N
    a.chunk_size = int(chunk_size)
    a.num_seqs = S
    a.num_chunks = Cn
    a.in_dtype = _dtype_code(x)
    a.a_kind = _abi.SSD_A_DIAG if diag else _abi.SSD_A_SCALAR
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
    return ck.keep(a)


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


def ssd_prefill_noalloc(x, dt, A, B, C, chunk_size: int, cu_seqlens, cu_chunk_seqlens, seq_idx,
                        last_chunk_indices, y, stream=None, **kw):
    """The prefill with its workspace in the library's static per-GPU array: this call and
    the library allocate nothing (``y`` and every other tensor come from the caller).
    Calls that overlap on one GPU race (see include/ssd.h).  Returns y."""
    args = prefill_args(x, dt, A, B, C, chunk_size, cu_seqlens, cu_chunk_seqlens, seq_idx,
                        last_chunk_indices, y, **kw)
    check("ssd_prefill_noalloc", lib().ssd_prefill_noalloc(ctypes.byref(args),
                                                           _stream_ptr(stream)))
    return y


def decode_args(x, dt, A, B, C, y, state_pool, state_indices, num_accepted_tokens=None,
                null_block_id: int = 0, D=None, dt_bias=None, dt_softplus: bool = False,
                dt_limit=(0.0, math.inf), device_error_flag=None,
                block_idx_last_computed=None, block_idx_last_scheduled=None) -> DecodeArgs:
    """Fill an ssd_decode_args.  Passing the two block index tensors selects the all cache
    mode: state_indices is then [B_pad, max_blocks] and ntok must be 1."""
    import torch
    ck = _Checker("ssd_state_update", x)
    if x.dim() != 4 or B.dim() != 4 or C.dim() != 4 or dt.dim() != 3 or y.dim() != 4:
        ck.fail("x, y must be [B_pad, ntok, H, P], dt [B_pad, ntok, H], B and C "
                "[B_pad, ntok, G, N]")
    B_pad, ntok, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    ck.t("x", x, _float_dtypes())
    for name, t in (("dt", dt), ("B", B), ("C", C), ("y", y)):
        ck.t(name, t, (x.dtype,))
    if tuple(dt.shape) != (B_pad, ntok, H) or tuple(y.shape) != tuple(x.shape) or \
            tuple(B.shape[:2]) != (B_pad, ntok) or tuple(C.shape) != tuple(B.shape):
        ck.fail("dt, B, C and y must match x's rows, tokens and heads")
    for name, t in (("x", x), ("dt", dt), ("B", B), ("C", C), ("y", y),
                    ("state_indices", state_indices)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    diag = A.dim() == 2
    ck.f32("A", A, numel=H * N if diag else H)
    ck.f32("D", D, numel=H)
    ck.f32("dt_bias", dt_bias, numel=H)
    ck.t("state_pool", state_pool, _pool_dtypes())
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, P, N) or \
            tuple(state_pool.stride()[1:]) != (P * N, N, 1):
        ck.fail("state_pool must be [slots, H, P, N] with contiguous slots")
    ck.t("state_indices", state_indices, (torch.int32,))
    if state_indices.dim() != 2 or state_indices.shape[0] != B_pad or \
            (block_idx_last_scheduled is None and state_indices.shape[1] != ntok):
        ck.fail("state_indices must be [B_pad, ntok] (or [B_pad, max_blocks] in the all "
                "cache mode)")
    ck.i32("num_accepted_tokens", num_accepted_tokens, numel=B_pad)
    ck.i32("block_idx_last_computed", block_idx_last_computed, numel=B_pad)
    ck.i32("block_idx_last_scheduled", block_idx_last_scheduled, numel=B_pad)
    ck.i32("device_error_flag", device_error_flag, min_numel=1)
    ck.gpu("x", x)     # every other tensor is on x's device
    device_error_flag = _flag_for(ck, device_error_flag)
    a = DecodeArgs()
    a.B_pad, a.ntok, a.H, a.P, a.G, a.N = B_pad, ntok, H, P, G, N
    a.in_dtype = _dtype_code(x)
    a.a_kind = _abi.SSD_A_DIAG if diag else _abi.SSD_A_SCALAR
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
    return ck.keep(a)


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
    ck = _Checker("ssd_conv1d_prefill", x)
    if x.dim() != 2 or out.dim() != 2 or weight.dim() != 2:
        ck.fail("x and out must be [T, D], weight [D, W]")
    T, D = x.shape
    ck.t("x", x, _float_dtypes())
    ck.t("out", out, (x.dtype,))
    if tuple(out.shape) != (T, D) or weight.shape[0] != D:
        ck.fail("out must match x, weight must have D rows")
    for name, t in (("x", x), ("out", out)):
        if t.stride(1) != 1:
            raise ValueError(f"{name}: each token row must be contiguous")
    if not weight.is_contiguous():
        raise ValueError("weight must be contiguous")
    S = cu_seqlens.numel() - 1
    ck.f32("weight", weight)
    ck.f32("bias", bias, numel=D)
    ck.i32("cu_seqlens", cu_seqlens)
    ck.i32("cu_chunk_seqlens", cu_chunk_seqlens, numel=seq_idx.numel() + 1)
    ck.i32("seq_idx", seq_idx)
    if conv_states is not None:
        ck.t("conv_states", conv_states, (x.dtype,))
        if conv_states.dim() != 3 or not conv_states[0].is_contiguous():
            ck.fail("conv_states must be [slots, W-1, D] or [slots, D, W-1] with contiguous "
                    "slots")
    ck.i32("state_indices", state_indices, numel=S)
    ck.i32("has_initial_state", has_initial_state, numel=S)
    ck.i32("device_error_flag", device_error_flag, min_numel=1)
    ck.gpu("x", x)     # every other tensor is on x's device
    device_error_flag = _flag_for(ck, device_error_flag)
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
    return ck.keep(a)


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
    ck = _Checker("ssd_conv1d_update", x)
    if x.dim() != 3 or out.dim() != 3 or weight.dim() != 2:
        ck.fail("x and out must be [B_pad, ntok, D], weight [D, W]")
    B_pad, ntok, D = x.shape
    ck.t("x", x, _float_dtypes())
    ck.t("out", out, (x.dtype,))
    if tuple(out.shape) != tuple(x.shape) or weight.shape[0] != D:
        ck.fail("out must match x, weight must have D rows")
    for name, t in (("x", x), ("out", out), ("weight", weight),
                    ("state_indices", state_indices)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    ck.f32("weight", weight)
    ck.f32("bias", bias, numel=D)
    ck.t("conv_states", conv_states, (x.dtype,))
    if conv_states.dim() != 3 or not conv_states[0].is_contiguous():
        ck.fail("conv_states must be [slots, W-1, D] or [slots, D, W-1] with contiguous slots")
    ck.i32("state_indices", state_indices, numel=B_pad)
    ck.i32("device_error_flag", device_error_flag, min_numel=1)
    ck.gpu("x", x)     # every other tensor is on x's device
    device_error_flag = _flag_for(ck, device_error_flag)
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
    return ck.keep(a)


def ssd_conv1d_update(x, weight, bias, conv_states, state_indices, out=None, stream=None,
                      **kw):
    """One decode step of the conv, in place on ``conv_states``.  Returns out."""
    import torch
    if out is None:
        out = torch.empty_like(x)
    args = conv1d_update_args(x, weight, bias, out, conv_states, state_indices, **kw)
    check("ssd_conv1d_update", lib().ssd_conv1d_update(ctypes.byref(args), _stream_ptr(stream)))
    return out
