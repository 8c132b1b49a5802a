"""The Python binding's argument checks, on the CPU: every tensor is checked for the dtype,
layout, element count and device the C ABI assumes before any pointer reaches the
library, so a host pointer, int64 metadata, a bool mask or a mismatched dtype raises
ValueError instead of being misread by a kernel.  (CPU tensors stand in for device ones:
a call whose tensors pass every other check stops at the GPU check.)"""
import pytest
import torch

from selective_state_space_mamba2_amd import api

T, H, P, G, N, S, CN, CS = 64, 4, 16, 2, 16, 2, 3, 32


def _prefill(**over):
    bf = torch.bfloat16
    kw = dict(x=torch.zeros(T, H, P, dtype=bf), dt=torch.zeros(T, H, dtype=bf),
              A=torch.zeros(H), B=torch.zeros(T, G, N, dtype=bf),
              C=torch.zeros(T, G, N, dtype=bf), chunk_size=CS,
              cu_seqlens=torch.zeros(S + 1, dtype=torch.int32),
              cu_chunk_seqlens=torch.zeros(CN + 1, dtype=torch.int32),
              seq_idx=torch.zeros(CN, dtype=torch.int32),
              last_chunk_indices=torch.zeros(S, dtype=torch.int32),
              y=torch.zeros(T, H, P, dtype=bf), D=torch.zeros(H),
              state_pool=torch.zeros(5, H, P, N), state_indices=torch.zeros(S, dtype=torch.int32),
              has_initial_state=torch.ones(S, dtype=torch.int32),
              chunk_states_out=torch.zeros(CN, H, P, N),
              device_error_flag=torch.zeros(1, dtype=torch.int32))
    kw.update(over)
    return kw


def _run_prefill(**over):
    kw = _prefill(**over)
    api.prefill_args(**kw)


def test_prefill_stops_at_the_gpu_check():
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        _run_prefill()


@pytest.mark.parametrize("over,match", [
    (dict(cu_seqlens=torch.zeros(S + 1, dtype=torch.int64)), "cu_seqlens has dtype"),
    (dict(seq_idx=torch.zeros(CN, dtype=torch.int64)), "seq_idx has dtype"),
    (dict(has_initial_state=torch.ones(S, dtype=torch.bool)), "has_initial_state has dtype"),
    (dict(state_indices=torch.zeros(S, dtype=torch.int64)), "state_indices has dtype"),
    (dict(dt=torch.zeros(T, H)), "dt has dtype"),
    (dict(B=torch.zeros(T, G, N)), "B has dtype"),
    (dict(y=torch.zeros(T, H, P)), "y has dtype"),
    (dict(A=torch.zeros(H, dtype=torch.bfloat16)), "A has dtype"),
    (dict(D=torch.zeros(H, dtype=torch.float64)), "D has dtype"),
    (dict(A=torch.zeros(H + 1)), "A has"),
    (dict(last_chunk_indices=torch.zeros(S + 1, dtype=torch.int32)), "last_chunk_indices has"),
    (dict(cu_chunk_seqlens=torch.zeros(CN, dtype=torch.int32)), "cu_chunk_seqlens has"),
    (dict(chunk_states_out=torch.zeros(CN, H, P, N + 1)), "chunk_states_out has"),
    (dict(state_pool=torch.zeros(5, H, P, N, dtype=torch.float64)), "state_pool has dtype"),
    (dict(state_pool=torch.zeros(5, H, N, P).transpose(2, 3)), "state_pool must be"),
    (dict(cu_seqlens=torch.zeros(2 * (S + 1), dtype=torch.int32)[::2]), "must be contiguous"),
    (dict(device_error_flag=torch.zeros(1, dtype=torch.int64)), "device_error_flag has dtype"),
    (dict(x=torch.zeros(T, H, P, dtype=torch.float16), dt=torch.zeros(T, H, dtype=torch.float16),
          B=torch.zeros(T, G, N, dtype=torch.float16), C=torch.zeros(T, G, N, dtype=torch.float16),
          y=torch.zeros(T, H, P, dtype=torch.float16)), "x has dtype"),
    (dict(D=torch.zeros(H, device="meta")), "D is on meta"),
    (dict(dt=torch.zeros(T, H + 1, dtype=torch.bfloat16)), "must match x"),
])
def test_prefill_argument_checks(over, match):
    with pytest.raises(ValueError, match=match):
        _run_prefill(**over)


def _decode(**over):
    bf = torch.bfloat16
    Bp, nt = 4, 2
    kw = dict(x=torch.zeros(Bp, nt, H, P, dtype=bf), dt=torch.zeros(Bp, nt, H, dtype=bf),
              A=torch.zeros(H), B=torch.zeros(Bp, nt, G, N, dtype=bf),
              C=torch.zeros(Bp, nt, G, N, dtype=bf), y=torch.zeros(Bp, nt, H, P, dtype=bf),
              state_pool=torch.zeros(9, H, P, N),
              state_indices=torch.zeros(Bp, nt, dtype=torch.int32),
              num_accepted_tokens=torch.ones(Bp, dtype=torch.int32), D=torch.zeros(H))
    kw.update(over)
    return kw


def test_decode_stops_at_the_gpu_check():
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        api.decode_args(**_decode())


@pytest.mark.parametrize("over,match", [
    (dict(state_indices=torch.zeros(4, 2, dtype=torch.int64)), "state_indices has dtype"),
    (dict(num_accepted_tokens=torch.ones(4, dtype=torch.int64)), "num_accepted_tokens has dtype"),
    (dict(num_accepted_tokens=torch.ones(3, dtype=torch.int32)), "num_accepted_tokens has"),
    (dict(state_indices=torch.zeros(4, 3, dtype=torch.int32)), "state_indices must be"),
    (dict(A=torch.zeros(H, dtype=torch.float64)), "A has dtype"),
    (dict(C=torch.zeros(4, 2, G, N)), "C has dtype"),
    (dict(state_pool=torch.zeros(9, H, P, N, dtype=torch.float64)), "state_pool has dtype"),
    (dict(D=torch.zeros(H, device="meta")), "D is on meta"),
])
def test_decode_argument_checks(over, match):
    with pytest.raises(ValueError, match=match):
        api.decode_args(**_decode(**over))


def _conv(**over):
    bf = torch.bfloat16
    D, W = 16, 4
    kw = dict(x=torch.zeros(T, D, dtype=bf), weight=torch.zeros(D, W), bias=torch.zeros(D),
              out=torch.zeros(T, D, dtype=bf), cu_seqlens=torch.zeros(S + 1, dtype=torch.int32),
              cu_chunk_seqlens=torch.zeros(CN + 1, dtype=torch.int32),
              seq_idx=torch.zeros(CN, dtype=torch.int32),
              conv_states=torch.zeros(5, W - 1, D, dtype=bf),
              state_indices=torch.zeros(S, dtype=torch.int32),
              has_initial_state=torch.zeros(S, dtype=torch.int32))
    kw.update(over)
    return kw


def test_conv_stops_at_the_gpu_check():
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        api.conv1d_args(**_conv())


@pytest.mark.parametrize("over,match", [
    (dict(weight=torch.zeros(16, 4, dtype=torch.bfloat16)), "weight has dtype"),
    (dict(cu_seqlens=torch.zeros(S + 1, dtype=torch.int64)), "cu_seqlens has dtype"),
    (dict(has_initial_state=torch.zeros(S, dtype=torch.bool)), "has_initial_state has dtype"),
    (dict(conv_states=torch.zeros(5, 3, 16)), "conv_states has dtype"),
    (dict(out=torch.zeros(T, 16)), "out has dtype"),
])
def test_conv_argument_checks(over, match):
    with pytest.raises(ValueError, match=match):
        api.conv1d_args(**_conv(**over))


def test_conv_update_checks():
    bf = torch.bfloat16
    kw = dict(x=torch.zeros(4, 1, 16, dtype=bf), weight=torch.zeros(16, 4), bias=None,
              out=torch.zeros(4, 1, 16, dtype=bf), conv_states=torch.zeros(5, 3, 16, dtype=bf),
              state_indices=torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        api.conv1d_update_args(**kw)
    with pytest.raises(ValueError, match="state_indices has dtype"):
        api.conv1d_update_args(**{**kw, "state_indices": torch.zeros(4, dtype=torch.int64)})


def test_device_error_names():
    assert api.device_error_names(0) == []
    assert api.device_error_names(2 | 8) == ["SLOT_RANGE", "CHAIN_WAIT"]
