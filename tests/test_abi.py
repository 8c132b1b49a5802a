"""The C ABI on the CPU: every declared symbol is exported, the ctypes mirror matches the
header's struct layout, and every host-side check returns its status before any launch
(the fake device pointers used here are never dereferenced)."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from selective_state_space_mamba2_amd import _abi
from selective_state_space_mamba2_amd._abi import DecodeArgs, PrefillArgs, lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(ssd_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_every_declared_function_is_exported():
    names = _declared_functions()
    assert set(names) == set(_abi.EXPORTS), names
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for n in names:
        assert n in exported, n
        getattr(lib(), n)


def test_abi_version_and_status_strings():
    assert lib().ssd_abi_version() == 3
    for s in range(8):
        assert lib().ssd_status_string(s)
    assert lib().ssd_status_string(99) == b"unknown status"


def _c_layout(struct_name, fields):
    src = ['#include <stdio.h>', '#include <stddef.h>', '#include "ssd.h"', 'int main(void){',
           f'printf("%zu\\n", sizeof({struct_name}));']
    for f in fields:
        src.append(f'printf("%zu\\n", offsetof({struct_name}, {f}));')
    src.append("return 0;}")
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "l.c")
        open(c, "w").write("\n".join(src))
        exe = os.path.join(d, "l")
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        return [int(v) for v in subprocess.run([exe], capture_output=True, text=True,
                                               check=True).stdout.split()]


@pytest.mark.parametrize("struct,cls", [("ssd_prefill_args", PrefillArgs),
                                        ("ssd_decode_args", DecodeArgs),
                                        ("ssd_conv1d_args", _abi.Conv1dArgs),
                                        ("ssd_conv1d_update_args", _abi.Conv1dUpdateArgs)])
def test_struct_layout_matches_header(struct, cls):
    names = [f[0] for f in cls._fields_]
    got = _c_layout(struct, names)
    assert got[0] == ctypes.sizeof(cls)
    for name, off in zip(names, got[1:]):
        assert getattr(cls, name).offset == off, name


# ----------------------------------------------------------------------------------------
# host-side validation (no launch happens for any of these)
# ----------------------------------------------------------------------------------------
FAKE = 0x10000   # a 256-byte aligned non-null "device" address; never dereferenced


def _good_prefill(**over):
    a = PrefillArgs()
    a.T, a.H, a.P, a.G, a.N, a.chunk_size = 512, 8, 64, 2, 128, 256
    a.num_seqs, a.num_chunks = 2, 3
    a.in_dtype, a.a_kind = _abi.SSD_BF16, _abi.SSD_A_SCALAR
    a.x = a.dt = a.B = a.C = a.y = a.A = FAKE
    a.x_stride_t = a.y_stride_t = 8 * 64
    a.dt_stride_t = 8
    a.bc_stride_t = 2 * 128
    a.cu_seqlens = a.cu_chunk_seqlens = a.seq_idx = a.last_chunk_indices = FAKE
    a.dt_min, a.dt_max = 0.0, float("inf")
    for k, v in over.items():
        setattr(a, k, v)
    return a


def _ws(a):
    n = ctypes.c_size_t(0)
    return lib().ssd_prefill_workspace_size(ctypes.byref(a), ctypes.byref(n)), n.value


def _al(v):
    return (v + 255) // 256 * 256


def test_workspace_size_layout():
    C, H, P, N, G, cs = 3, 8, 64, 128, 2, 256
    # per (chunk, group) in the input dtype, shared by the heads of a group: the C.B^T
    # fragments of the 16 row tiles (tile i needs i//2 + 1 fragments of 512 values) and
    # B^T; per (chunk, head) fp32: the cumsum of delta*A and delta; per (chunk, group): the
    # C rows as fragments
    nfrag = sum(i // 2 + 1 for i in range(cs // 16))
    assert nfrag == 72
    S = 2
    prep = (_al(C * G * nfrag * 512 * 2) + _al(C * G * N * cs * 2) + _al(C * G * cs * N * 2)
            + _al(S * 4))
    # the chunk-chain kernel (bf16, head dim 64) forms delta and the cumsum itself, and has
    # per (chunk, head) an int32 flag for each of its 4 wavefronts, per chunk its dispatch
    # row, and without a chunk-state output a two-deep fp32 state ring per (sequence, head)
    chain = _al(C * H * 4 * 4) + _al(C * 4)
    ring = _al(S * H * 2 * P * N * 4)
    for over, extra in (({}, ring), (dict(chunk_states_out=FAKE), 0),
                        (dict(chunk_states_out=FAKE, has_initial_state=FAKE, state_pool=FAKE,
                              state_indices=FAKE, num_slots=4, slot_stride=8 * 64 * 128), 0)):
        st, n = _ws(_good_prefill(**over))
        assert st == 0 and n == prep + chain + extra
    # fp32 inputs run the march kernel: no chain buffers
    st, n = _ws(_good_prefill(in_dtype=_abi.SSD_F32, chunk_size=64))
    nf64 = sum(i // 2 + 1 for i in range(64 // 16))
    C64 = 3
    assert st == 0 and n == (_al(C64 * G * nf64 * 512 * 4) + _al(C64 * G * N * 64 * 4)
                             + _al(C64 * H * 2 * 64 * 4) + _al(C64 * G * 64 * N * 4) + _al(S * 4))
    st, n = _ws(_good_prefill(a_kind=_abi.SSD_A_DIAG, H=64, P=1, G=1, N=16, x_stride_t=64,
                              y_stride_t=64, dt_stride_t=64, bc_stride_t=16))
    assert st == 0 and n == 0
    # the all cache mode adds one int32 per chunk: the pool slot of its end state
    st, n = _ws(_good_prefill(chunk_states_out=FAKE, **_ALL_MODE))
    assert st == 0 and n == prep + chain + _al(C * 4)


_ALL_MODE = dict(block_size=512, idx_stride=6, num_computed=FAKE, state_pool=FAKE,
                 state_indices=FAKE, num_slots=16, slot_stride=8 * 64 * 128)


@pytest.mark.parametrize("over,status", [
    (dict(), _abi.SSD_OK),
    (dict(block_size=-1), _abi.SSD_ERR_BAD_SHAPE),
    (dict(block_size=384), _abi.SSD_ERR_BAD_SHAPE),            # not a multiple of chunk_size
    (dict(idx_stride=0), _abi.SSD_ERR_BAD_SHAPE),
    (dict(num_computed=None), _abi.SSD_ERR_NULL_POINTER),
    (dict(state_indices=None), _abi.SSD_ERR_NULL_POINTER),
    (dict(has_initial_state=FAKE), _abi.SSD_ERR_NULL_POINTER),  # needs block_idx_last_computed
    (dict(has_initial_state=FAKE, block_idx_last_computed=FAKE), _abi.SSD_OK),
    (dict(write_final_to_pool=1), _abi.SSD_ERR_NULL_POINTER),   # needs block_idx_last_scheduled
    (dict(write_final_to_pool=1, block_idx_last_scheduled=FAKE), _abi.SSD_OK),
])
def test_prefill_all_cache_mode_host_checks(over, status):
    assert _ws(_good_prefill(**{**_ALL_MODE, **over}))[0] == status


def test_prefill_all_cache_mode_with_diagonal_a():
    """The Mamba1 scan takes the all cache mode too; it resolves block entries itself, so it
    needs no workspace."""
    diag = dict(a_kind=_abi.SSD_A_DIAG, H=64, P=1, G=1, N=16, x_stride_t=64, y_stride_t=64,
                dt_stride_t=64, bc_stride_t=16, chunk_size=256, slot_stride=64 * 16)
    assert _ws(_good_prefill(**{**_ALL_MODE, **diag})) == (_abi.SSD_OK, 0)
    assert _ws(_good_prefill(**{**_ALL_MODE, **diag, "block_size": 384}))[0] == _abi.SSD_ERR_BAD_SHAPE


def test_kernel_count():
    n = ctypes.c_int32(-1)
    names = (ctypes.c_char_p * _abi.SSD_PREFILL_MAX_KERNELS)()
    assert lib().ssd_prefill_kernel_count(ctypes.byref(_good_prefill()), ctypes.byref(n), names) == 0
    assert n.value == 2
    assert [names[i] for i in range(2)] == [b"k_chunk_prep", b"k_chunk_chain"]
    f32 = _good_prefill(in_dtype=_abi.SSD_F32, chunk_size=64)
    assert lib().ssd_prefill_kernel_count(ctypes.byref(f32), ctypes.byref(n), names) == 0
    assert n.value == 2 and [names[i] for i in range(2)] == [b"k_chunk_prep", b"k_chunk_march"]
    diag = _good_prefill(a_kind=_abi.SSD_A_DIAG, H=64, P=1, G=1, N=16, x_stride_t=64,
                         y_stride_t=64, dt_stride_t=64, bc_stride_t=16)
    assert lib().ssd_prefill_kernel_count(ctypes.byref(diag), ctypes.byref(n), names) == 0
    # 64 channels in a small batch: two 32-channel workgroups per sequence beat one of 64
    assert n.value == 1 and names[0] == b"k_diag_scan_mixed"
    diag.H = 200   # 2 + 3 workgroups per sequence would not shorten the launch
    diag.x_stride_t = diag.y_stride_t = diag.dt_stride_t = 200
    assert lib().ssd_prefill_kernel_count(ctypes.byref(diag), ctypes.byref(n), names) == 0
    assert n.value == 1 and names[0] == b"k_diag_scan"
    empty = _good_prefill(T=0, num_seqs=0, num_chunks=0)
    assert lib().ssd_prefill_kernel_count(ctypes.byref(empty), ctypes.byref(n), None) == 0
    assert n.value == 0


@pytest.mark.parametrize("S,H,mixed", [
    (8, 5120, True),    # 640 workgroups of 64 channels on 256 CUs: 3 passes on half the CUs
    (4, 5120, True),    # the shapes of the mixed-grid GPU tests
    (7, 2312, True),
    (6, 72, True),
    (1, 200, False),    # 2 + 3 workgroups: no shorter than the 4 of 64 channels
    (3, 5000, False),   # uniform grid in one pass; mixed needs two
])
def test_diag_grid_choice(S, H, mixed):
    """The Mamba1 scan's grid as the host picks it on a 256-CU device (the count the
    library assumes without one): the kernel name ssd_prefill_kernel_count reports."""
    n = ctypes.c_int32(-1)
    names = (ctypes.c_char_p * _abi.SSD_PREFILL_MAX_KERNELS)()
    a = _good_prefill(a_kind=_abi.SSD_A_DIAG, H=H, P=1, G=1, N=16, num_seqs=S, num_chunks=S,
                      T=64 * S, chunk_size=64, x_stride_t=H, y_stride_t=H, dt_stride_t=H,
                      bc_stride_t=16)
    assert lib().ssd_prefill_kernel_count(ctypes.byref(a), ctypes.byref(n), names) == 0
    assert n.value == 1
    assert names[0] == (b"k_diag_scan_mixed" if mixed else b"k_diag_scan")


@pytest.mark.parametrize("over,status", [
    (dict(H=6, G=4), _abi.SSD_ERR_BAD_SHAPE),             # H % G != 0
    (dict(P=0), _abi.SSD_ERR_BAD_SHAPE),
    (dict(chunk_size=0), _abi.SSD_ERR_BAD_SHAPE),
    (dict(in_dtype=7), _abi.SSD_ERR_BAD_SHAPE),
    (dict(a_kind=5), _abi.SSD_ERR_BAD_SHAPE),
    (dict(state_dtype=3), _abi.SSD_ERR_BAD_SHAPE),
    (dict(in_dtype=_abi.SSD_F16), _abi.SSD_ERR_BAD_SHAPE),       # fp16 is a pool type only
    (dict(num_chunks=1), _abi.SSD_ERR_BAD_SHAPE),         # fewer chunks than sequences
    (dict(num_chunks=600), _abi.SSD_ERR_BAD_SHAPE),       # more chunks than tokens
    (dict(T=1), _abi.SSD_ERR_BAD_SHAPE),                  # fewer tokens than sequences
    (dict(x_stride_t=100), _abi.SSD_ERR_BAD_SHAPE),
    (dict(dt_stride_t=4), _abi.SSD_ERR_BAD_SHAPE),
    (dict(bc_stride_t=128), _abi.SSD_ERR_BAD_SHAPE),
    (dict(dt_min=1.0, dt_max=0.5), _abi.SSD_ERR_BAD_SHAPE),
    (dict(dt_min=float("nan")), _abi.SSD_ERR_BAD_SHAPE),
    (dict(x=None), _abi.SSD_ERR_NULL_POINTER),
    (dict(A=None), _abi.SSD_ERR_NULL_POINTER),
    (dict(seq_idx=None), _abi.SSD_ERR_NULL_POINTER),
    (dict(has_initial_state=FAKE), _abi.SSD_ERR_NULL_POINTER),   # no pool given
    (dict(write_final_to_pool=1, state_pool=FAKE), _abi.SSD_ERR_NULL_POINTER),  # no indices
    (dict(state_pool=FAKE, state_indices=FAKE, num_slots=0), _abi.SSD_ERR_BAD_SHAPE),
    (dict(state_pool=FAKE, state_indices=FAKE, num_slots=2, slot_stride=10),
     _abi.SSD_ERR_BAD_SHAPE),
    (dict(P=32), _abi.SSD_ERR_UNSUPPORTED),                # not instantiated
    (dict(chunk_size=100), _abi.SSD_ERR_UNSUPPORTED),
    (dict(in_dtype=_abi.SSD_F32, chunk_size=128), _abi.SSD_ERR_UNSUPPORTED),   # fp32 at cs=128
    (dict(a_kind=_abi.SSD_A_DIAG), _abi.SSD_ERR_BAD_SHAPE),    # diag needs P == 1
    (dict(dt_min=-1.0), _abi.SSD_ERR_UNSUPPORTED),          # chunked path needs delta >= 0
])
def test_prefill_host_checks(over, status):
    a = _good_prefill(**over)
    assert _ws(a)[0] == status
    assert lib().ssd_prefill(ctypes.byref(a), FAKE, 1 << 40, None) == status


def test_prefill_workspace_checks():
    a = _good_prefill()
    need = _ws(a)[1]
    assert lib().ssd_prefill(ctypes.byref(a), None, need, None) == _abi.SSD_ERR_WORKSPACE
    assert lib().ssd_prefill(ctypes.byref(a), FAKE, need - 1, None) == _abi.SSD_ERR_WORKSPACE
    assert lib().ssd_prefill(ctypes.byref(a), FAKE + 8, need, None) == _abi.SSD_ERR_WORKSPACE


def test_prefill_vector_access_checks():
    a = _good_prefill(x=FAKE + 2)            # x not 16-byte aligned
    assert lib().ssd_prefill(ctypes.byref(a), FAKE, 1 << 40, None) == _abi.SSD_ERR_UNSUPPORTED
    a = _good_prefill(x_stride_t=8 * 64 + 3)  # row stride breaks 16-byte alignment
    assert lib().ssd_prefill(ctypes.byref(a), FAKE, 1 << 40, None) == _abi.SSD_ERR_UNSUPPORTED


def test_prefill_empty_batch_is_a_noop():
    a = _good_prefill(T=0, num_seqs=0, num_chunks=0)
    assert _ws(a) == (0, 0)
    assert lib().ssd_prefill(ctypes.byref(a), None, 0, None) == 0
    assert lib().ssd_prefill(None, None, 0, None) == _abi.SSD_ERR_NULL_POINTER


def test_diag_host_checks():
    base = dict(a_kind=_abi.SSD_A_DIAG, H=64, P=1, G=1, N=16, x_stride_t=64, y_stride_t=64,
                dt_stride_t=64, bc_stride_t=16)
    assert _ws(_good_prefill(**base))[0] == 0
    assert _ws(_good_prefill(**{**base, "N": 32, "bc_stride_t": 32}))[0] == _abi.SSD_ERR_UNSUPPORTED
    assert _ws(_good_prefill(**base, dA_cumsum_out=FAKE))[0] == _abi.SSD_ERR_UNSUPPORTED


@pytest.mark.parametrize("in_dtype", [_abi.SSD_BF16, _abi.SSD_F32])
@pytest.mark.parametrize("P", [1, 16, 64])
@pytest.mark.parametrize("N", [16, 128])
@pytest.mark.parametrize("cs", [64, 256])
def test_minimum_instantiation_set_plans(in_dtype, P, N, cs):
    """Every (dtype, head_dim, dstate, chunk_size) of the minimum instantiation set has a
    kernel: head_dim 1 runs the sequential scan, the others the chunked kernels."""
    H, G = 8, 2
    a = _good_prefill(in_dtype=in_dtype, H=H, P=P, G=G, N=N, chunk_size=cs, x_stride_t=H * P,
                      y_stride_t=H * P, dt_stride_t=H, bc_stride_t=G * N)
    st, need = _ws(a)
    assert st == 0, (in_dtype, P, N, cs, st)
    n = ctypes.c_int32(-1)
    names = (ctypes.c_char_p * _abi.SSD_PREFILL_MAX_KERNELS)()
    assert lib().ssd_prefill_kernel_count(ctypes.byref(a), ctypes.byref(n), names) == 0
    if P == 1:
        assert need == 0 and n.value == 1 and names[0] == b"k_diag_scan"
    else:
        assert n.value == 2 and names[0] == b"k_chunk_prep"


def _good_decode(**over):
    a = DecodeArgs()
    a.B_pad, a.ntok, a.H, a.P, a.G, a.N = 8, 4, 48, 64, 4, 128
    a.in_dtype, a.a_kind = _abi.SSD_BF16, _abi.SSD_A_SCALAR
    a.x = a.dt = a.B = a.C = a.y = a.A = a.state_pool = a.state_indices = FAKE
    a.slot_stride, a.num_slots = 48 * 64 * 128, 16
    a.dt_min, a.dt_max = 0.0, float("inf")
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,status", [
    (dict(ntok=0), _abi.SSD_ERR_BAD_SHAPE),
    (dict(ntok=17), _abi.SSD_ERR_UNSUPPORTED),
    (dict(H=47), _abi.SSD_ERR_BAD_SHAPE),
    (dict(N=48), _abi.SSD_ERR_UNSUPPORTED),
    (dict(P=256), _abi.SSD_ERR_UNSUPPORTED),               # P*N above the per-head limit
    (dict(a_kind=_abi.SSD_A_DIAG), _abi.SSD_ERR_BAD_SHAPE),      # diag needs P == G == 1
    (dict(a_kind=_abi.SSD_A_DIAG, P=1, G=1, N=32, slot_stride=48 * 32), _abi.SSD_ERR_UNSUPPORTED),
    (dict(a_kind=7), _abi.SSD_ERR_BAD_SHAPE),
    (dict(state_dtype=3), _abi.SSD_ERR_BAD_SHAPE),
    (dict(in_dtype=3), _abi.SSD_ERR_BAD_SHAPE),
    (dict(state_pool=None), _abi.SSD_ERR_NULL_POINTER),
    (dict(state_indices=None), _abi.SSD_ERR_NULL_POINTER),
    (dict(slot_stride=100), _abi.SSD_ERR_BAD_SHAPE),
    (dict(num_slots=0), _abi.SSD_ERR_BAD_SHAPE),
    (dict(dt_min=2.0, dt_max=1.0), _abi.SSD_ERR_BAD_SHAPE),
    (dict(state_pool=FAKE + 4), _abi.SSD_ERR_UNSUPPORTED),
    (dict(state_dtype=_abi.SSD_BF16, slot_stride=48 * 64 * 128 + 4), _abi.SSD_ERR_UNSUPPORTED),
    (dict(state_dtype=_abi.SSD_F16, slot_stride=48 * 64 * 128 + 4), _abi.SSD_ERR_UNSUPPORTED),
    (dict(in_dtype=_abi.SSD_F16), _abi.SSD_ERR_BAD_SHAPE),       # fp16 is a pool type only
    (dict(idx_stride=-1), _abi.SSD_ERR_BAD_SHAPE),
    (dict(idx_stride=5), _abi.SSD_ERR_BAD_SHAPE),                # all cache mode needs ntok 1
    (dict(idx_stride=5, ntok=1, num_accepted_tokens=FAKE), _abi.SSD_ERR_BAD_SHAPE),
    (dict(idx_stride=5, ntok=1), _abi.SSD_ERR_NULL_POINTER),     # block index arrays missing
    (dict(idx_stride=5, ntok=1, block_idx_last_computed=FAKE), _abi.SSD_ERR_NULL_POINTER),
])
def test_decode_host_checks(over, status):
    a = _good_decode(**over)
    assert lib().ssd_state_update(ctypes.byref(a), None) == status


def test_decode_empty_batch_is_a_noop():
    assert lib().ssd_state_update(ctypes.byref(_good_decode(B_pad=0, x=None)), None) == 0


# ----------------------------------------------------------------------------------------
# conv1d host checks (no launch happens for any of these)
# ----------------------------------------------------------------------------------------
def _good_conv(**over):
    a = _abi.Conv1dArgs()
    a.T, a.D, a.W, a.num_seqs, a.num_chunks, a.in_dtype = 512, 3072, 4, 2, 3, _abi.SSD_BF16
    a.x = a.out = a.weight = a.cu_seqlens = a.cu_chunk_seqlens = a.seq_idx = FAKE
    a.x_stride_t = a.out_stride_t = 3072
    for k, v in over.items():
        setattr(a, k, v)
    return a


_CONV_POOL = dict(conv_states=FAKE, state_indices=FAKE, num_slots=8, slot_stride=3 * 3072)


@pytest.mark.parametrize("over,status", [
    (dict(T=-1), _abi.SSD_ERR_BAD_SHAPE),
    (dict(W=1), _abi.SSD_ERR_BAD_SHAPE),
    (dict(W=3), _abi.SSD_ERR_UNSUPPORTED),
    (dict(D=3076, x_stride_t=3076, out_stride_t=3076), _abi.SSD_ERR_UNSUPPORTED),
    (dict(in_dtype=5), _abi.SSD_ERR_BAD_SHAPE),
    (dict(activation=2), _abi.SSD_ERR_BAD_SHAPE),
    (dict(state_layout=2), _abi.SSD_ERR_BAD_SHAPE),
    (dict(num_chunks=1), _abi.SSD_ERR_BAD_SHAPE),            # fewer chunks than sequences
    (dict(x_stride_t=3000), _abi.SSD_ERR_BAD_SHAPE),
    (dict(x=None), _abi.SSD_ERR_NULL_POINTER),
    (dict(weight=None), _abi.SSD_ERR_NULL_POINTER),
    (dict(conv_states=FAKE), _abi.SSD_ERR_NULL_POINTER),     # a pool needs state_indices
    (dict(_CONV_POOL, slot_stride=3 * 3072 - 8), _abi.SSD_ERR_BAD_SHAPE),
    (dict(_CONV_POOL, num_slots=0), _abi.SSD_ERR_BAD_SHAPE),
    (dict(_CONV_POOL, conv_states=FAKE + 8), _abi.SSD_ERR_UNSUPPORTED),
    (dict(x=FAKE + 4), _abi.SSD_ERR_UNSUPPORTED),
    (dict(x_stride_t=3076), _abi.SSD_ERR_UNSUPPORTED),
    (dict(bias=FAKE + 4), _abi.SSD_ERR_UNSUPPORTED),
    # a wave's rows (T/8 + 1 of them) would span 2 GiB or more of x: 32-bit row offsets
    (dict(T=1 << 21, x_stride_t=8192, out_stride_t=8192), _abi.SSD_ERR_UNSUPPORTED),
])
def test_conv1d_prefill_host_checks(over, status):
    assert lib().ssd_conv1d_prefill(ctypes.byref(_good_conv(**over)), None) == status


def test_conv1d_prefill_empty_batch_is_a_noop():
    a = _good_conv(T=0, num_seqs=0, num_chunks=0, x=None)
    assert lib().ssd_conv1d_prefill(ctypes.byref(a), None) == _abi.SSD_OK


def _good_conv_update(**over):
    a = _abi.Conv1dUpdateArgs()
    a.B_pad, a.ntok, a.D, a.W, a.in_dtype = 8, 1, 3072, 4, _abi.SSD_BF16
    a.x = a.out = a.weight = a.conv_states = a.state_indices = FAKE
    a.num_slots, a.slot_stride = 16, 3 * 3072
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,status", [
    (dict(ntok=0), _abi.SSD_ERR_BAD_SHAPE),
    (dict(ntok=17), _abi.SSD_ERR_UNSUPPORTED),
    (dict(W=5), _abi.SSD_ERR_UNSUPPORTED),
    (dict(conv_states=None), _abi.SSD_ERR_NULL_POINTER),
    (dict(state_indices=None), _abi.SSD_ERR_NULL_POINTER),
    (dict(slot_stride=100), _abi.SSD_ERR_BAD_SHAPE),
    (dict(out=FAKE + 2), _abi.SSD_ERR_UNSUPPORTED),
    (dict(B_pad=0, x=None), _abi.SSD_OK),
])
def test_conv1d_update_host_checks(over, status):
    assert lib().ssd_conv1d_update(ctypes.byref(_good_conv_update(**over)), None) == status


def test_probe_stream_host_checks():
    f = lib().ssd_probe_stream
    assert f(FAKE, 16, FAKE, 16, None, 0, None) == _abi.SSD_ERR_NULL_POINTER   # no sink
    assert f(None, 16, FAKE, 0, FAKE, 0, None) == _abi.SSD_ERR_NULL_POINTER
    assert f(FAKE, 15, FAKE, 16, FAKE, 0, None) == _abi.SSD_ERR_BAD_SHAPE
    assert f(FAKE + 4, 16, FAKE, 16, FAKE, 0, None) == _abi.SSD_ERR_UNSUPPORTED
    assert f(FAKE, (1 << 35) + 16, FAKE, 0, FAKE, 0, None) == _abi.SSD_ERR_BAD_SHAPE
    assert f(FAKE, 16, FAKE, 16, FAKE, 12, None) == _abi.SSD_ERR_BAD_SHAPE    # no such form
    assert f(FAKE, 16, FAKE, 16, FAKE, -1, None) == _abi.SSD_ERR_BAD_SHAPE
    assert f(None, 0, None, 0, FAKE, 11, None) == 0                           # nothing to move


def test_prefill_noalloc_host_checks():
    """The allocation-free prefill returns the same host-check statuses as ssd_prefill, and
    SSD_ERR_WORKSPACE when the workspace needed exceeds the static array (before any device
    call)."""
    f = lib().ssd_prefill_noalloc
    assert f(None, None) == _abi.SSD_ERR_NULL_POINTER
    assert f(ctypes.byref(_good_prefill(P=32)), None) == _abi.SSD_ERR_UNSUPPORTED
    assert f(ctypes.byref(_good_prefill(x=None)), None) == _abi.SSD_ERR_NULL_POINTER
    big = _good_prefill(T=1 << 19, num_chunks=2048)
    st, need = _ws(big)
    assert st == 0 and need > _abi.SSD_NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(big), None) == _abi.SSD_ERR_WORKSPACE
    assert f(ctypes.byref(_good_prefill(T=0, num_seqs=0, num_chunks=0)), None) == 0
