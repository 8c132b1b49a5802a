"""The allocation-free prefill (ssd_prefill_noalloc) against ssd_prefill, through the C ABI.

Two calls in a row share the GPU's static workspace array: a larger batch (three varlen
sequences, pool gather and write-back, every chunk-end state), then a smaller one whose
chain hands its state through the workspace ring (no chunk-state output) in what the first
call left behind.  Each call's y, chunk states and pool must equal what ssd_prefill gives
on the same inputs with a workspace of its own (same kernels, so bit for bit; at least to
the input dtype's tolerance)."""
import pytest
import torch

from gpu_helpers import TOL, assert_close, dev_f32, dev_i32, dev_token, prefill_metadata
from selective_state_space_mamba2_amd import api
from selective_state_space_mamba2_amd.inputs import make_prefill

pytestmark = pytest.mark.gpu


def _run(inp, noalloc, want_states):
    cuc, sidx, last = prefill_metadata(inp)
    x, dt, B, C = (dev_token(inp, n) for n in ("x", "dt", "B", "C"))
    y = torch.full_like(x, float("nan"))
    pool = torch.from_numpy(inp.pool).cuda()
    states = (torch.full((len(sidx), inp.H, inp.P, inp.N), float("nan"), device="cuda")
              if want_states else None)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    kw = dict(D=dev_f32(inp.D), state_pool=pool, state_indices=dev_i32(inp.state_indices),
              has_initial_state=dev_i32(inp.has_initial_state), write_final_to_pool=True,
              chunk_states_out=states, device_error_flag=flag)
    md = (dev_i32(inp.cu_seqlens), dev_i32(cuc), dev_i32(sidx), dev_i32(last))
    if noalloc:
        api.ssd_prefill_noalloc(x, dt, dev_f32(inp.A), B, C, inp.chunk_size, *md, y, **kw)
    else:
        api.ssd_prefill(x, dt, dev_f32(inp.A), B, C, inp.chunk_size, *md, y=y, **kw)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    return y, states, pool


def _compare(inp, want_states):
    ref = _run(inp, False, want_states)
    got = _run(inp, True, want_states)
    tol = TOL[inp.in_dtype]
    for what, g, r in zip(("y", "chunk states", "pool"), got, ref):
        if r is None:
            continue
        assert_close(g.float().cpu().numpy(), r.float().cpu().numpy(), tol, what)
        assert torch.equal(g, r), f"{what} differs from ssd_prefill's"


def test_noalloc_matches_prefill_twice_then_smaller():
    big = make_prefill(90, in_dtype="bf16", H=16, P=64, G=2, N=128, chunk_size=256,
                       lengths=[3 * 256 + 17, 300, 2 * 256 - 1], num_computed=[0, 11, 7],
                       init="pool", pool_slots=16)
    _compare(big, want_states=True)
    small = make_prefill(91, in_dtype="bf16", H=8, P=64, G=1, N=128, chunk_size=256,
                         lengths=[5 * 256 - 3], num_computed=[40], init="pool", pool_slots=4)
    _compare(small, want_states=False)
