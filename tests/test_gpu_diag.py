"""GPU parity of the Mamba1-style diagonal selective scan (A[channel, state], P = 1)."""
import numpy as np
import pytest

from gpu_helpers import TOL, assert_close, check_prefill, oracle_prefill, run_prefill
from selective_state_space_mamba2_amd.inputs import make_prefill, workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_diag_with_pool_and_checkpoints(dtype):
    """200 channels (a ragged last block of 64), three sequences with unaligned resume
    points, two of them starting from pool states."""
    inp = make_prefill(40, in_dtype=dtype, H=200, P=1, G=1, N=16, chunk_size=128,
                       lengths=[300, 77, 1000], num_computed=[0, 5, 130], a_kind="diag",
                       init="pool", pool_slots=8)
    inp.has_initial_state[1] = 0
    got = run_prefill(inp)
    assert got["flag"] == 0
    check_prefill(inp, got, oracle_prefill(inp))
    owned = set(int(v) for v in inp.state_indices)
    for s in range(8):
        if s not in owned:
            np.testing.assert_array_equal(got["pool"][s], inp.pool[s])


@pytest.mark.parametrize("pool", ["bf16", "f16"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_diag_2byte_state_pool(dtype, pool):
    """The Mamba1 scan gathering from and writing back to a bf16 or fp16 pool."""
    from gpu_helpers import pool_tol, rounded_pool
    inp = rounded_pool(make_prefill(43, in_dtype=dtype, H=200, P=1, G=1, N=16, chunk_size=128,
                                    lengths=[300, 77], num_computed=[0, 5], a_kind="diag",
                                    init="pool", pool_slots=8), pool)
    got = run_prefill(inp)
    assert got["flag"] == 0
    check_prefill(inp, got, oracle_prefill(inp), pool_tol=pool_tol(inp))
    owned = set(int(v) for v in inp.state_indices)
    for s in range(8):
        if s not in owned:
            np.testing.assert_array_equal(got["pool"][s], inp.pool[s])


@pytest.mark.parametrize("H", [100, 36])
def test_diag_bf16_element_path(H):
    """bf16 inputs the 16-byte tile path cannot take (channel counts that are not whole
    8-channel groups, so the token strides are not multiples of 8 either): one element per
    access, the same results."""
    inp = make_prefill(44, in_dtype="bf16", H=H, P=1, G=1, N=16, chunk_size=64,
                       lengths=[150, 77], num_computed=[0, 9], a_kind="diag",
                       init="pool", pool_slots=4)
    got = run_prefill(inp)
    assert got["flag"] == 0
    check_prefill(inp, got, oracle_prefill(inp))


def test_diag_bf16_tile_path_with_projection_views():
    """x, B and C as views into one projection buffer (token strides 112, dt and y strides
    72, all multiples of 8): the 16-byte tile path with strides other than the width."""
    inp = make_prefill(45, in_dtype="bf16", H=64, P=1, G=1, N=16, chunk_size=64,
                       lengths=[150, 77], num_computed=[0, 9], a_kind="diag",
                       init="pool", pool_slots=4)
    got = run_prefill(inp, views=True)
    assert got["flag"] == 0
    check_prefill(inp, got, oracle_prefill(inp))


def test_diag_several_checkpoints_per_token_tile():
    """chunk_size 24 with unaligned resume points: several chunk ends fall inside one
    32-token tile of the scan, so groups of tokens restart at unaligned positions."""
    inp = make_prefill(42, in_dtype="bf16", H=72, P=1, G=1, N=16, chunk_size=24,
                       lengths=[97, 33, 150], num_computed=[0, 7, 50], a_kind="diag",
                       init="pool", pool_slots=4)
    got = run_prefill(inp)
    assert got["flag"] == 0
    check_prefill(inp, got, oracle_prefill(inp))


@pytest.mark.parametrize("dtype,H", [("f32", 64), ("bf16", 64), ("bf16", 200)])
def test_diag_softplus_and_long_memory(dtype, H):
    """dt bias, softplus and a dt limit with slow decays (long memory): the element path
    (fp32), and the 16-byte path of the 32-channel (64 channels) and the 64-channel (200
    channels) workgroups, each with its own per-channel bias registers."""
    inp = make_prefill(41, in_dtype=dtype, H=H, P=1, G=1, N=16, chunk_size=64,
                       lengths=[500], a_kind="diag", A_range=(1e-3, 1e-2))
    bias = np.random.default_rng(1).normal(-1, 0.3, H).astype(np.float32).astype(np.float64)
    got = run_prefill(inp, dt_bias=bias, softplus=True, dt_limit=(0.0, 0.5))
    check_prefill(inp, got, oracle_prefill(inp, dt_bias=bias, softplus=True,
                                           dt_limit=(0.0, 0.5)))


def test_full_mamba1_long_diag():
    inp = workload("mamba1_long_diag")
    got = run_prefill(inp)
    assert got["flag"] == 0 and np.isfinite(got["y"]).all()
    assert len(got["metadata"][1]) == 64
    chans = [0, 2501, 5119]
    check_prefill(inp, got, oracle_prefill(inp, seqs=[3], heads=chans), heads=chans)


MIXED_SHAPES = {
    # 4 x 5120: 64 large and 32 small workgroups per sequence, the small ones paired in
    # whole runs of 16 workgroup ids
    "4x5120": ([150, 97, 130, 64], [0, 5, 60, 3], 5120),
    # 7 x 2312: 28 large and 17 small per sequence (pairs of small workgroups cross
    # sequence boundaries, 119 small ones leave a run of 7 unpaired; the last small
    # workgroup of a sequence holds 8 channels)
    "7x2312": ([70, 33, 96, 64, 1, 129, 40], [0, 7, 60, 3, 0, 1, 9], 2312),
    # 6 x 72: small workgroups only (3 per sequence, the third with 8 channels)
    "6x72": ([90, 64, 3, 130, 65, 20], [1, 0, 2, 63, 64, 0], 72),
}


@pytest.mark.parametrize("shape", sorted(MIXED_SHAPES))
@pytest.mark.parametrize("dtype,pool", [("bf16", "f32"), ("bf16", "bf16"), ("f32", "f16")])
def test_diag_mixed_workgroup_grid(dtype, pool, shape):
    """Mamba1 batches for which the host picks the grid of 64-channel workgroups with 4
    states per lane and 32-channel ones with 2 states per lane (on 256 CUs): every channel
    of both kinds, its checkpoints and its pool entries against the oracle."""
    from gpu_helpers import pool_tol, rounded_pool
    lengths, computed, H = MIXED_SHAPES[shape]
    inp = make_prefill(44, in_dtype=dtype, H=H, P=1, G=1, N=16, chunk_size=64,
                       lengths=lengths, num_computed=computed, a_kind="diag",
                       init="pool", pool_slots=2 * len(lengths))
    if pool != "f32":
        rounded_pool(inp, pool)
    got = run_prefill(inp)
    assert got["flag"] == 0
    check_prefill(inp, got, oracle_prefill(inp), pool_tol=pool_tol(inp))


@pytest.mark.parametrize("H,lengths,computed", [
    (5120, [150, 97, 130, 64], [0, 5, 60, 3]),    # the mixed grid
    (200, [150, 77], [0, 9]),                     # the uniform grid
])
def test_diag_graph_capture_and_replay(H, lengths, computed):
    """The Mamba1 scan captured in a HIP graph and replayed several times with eager work
    in between gives the eager call's y, checkpoints and pool on every replay."""
    import torch
    from gpu_helpers import dev_f32, dev_i32, dev_token, prefill_metadata
    from selective_state_space_mamba2_amd import api
    inp = make_prefill(46, in_dtype="bf16", H=H, P=1, G=1, N=16, chunk_size=64,
                       lengths=lengths, num_computed=computed, a_kind="diag", init="pool",
                       pool_slots=2 * len(lengths))
    cuc, sidx, last = prefill_metadata(inp)
    x, dt, B, C = (dev_token(inp, n) for n in ("x", "dt", "B", "C"))
    A, D = dev_f32(inp.A), dev_f32(inp.D)
    md = [dev_i32(inp.cu_seqlens), dev_i32(cuc), dev_i32(sidx), dev_i32(last)]
    pool0 = torch.from_numpy(inp.pool).cuda()
    pool = pool0.clone()
    y = torch.zeros_like(x)
    states = torch.zeros(len(sidx), H, 1, 16, device="cuda")
    kw = dict(y=y, D=D, state_pool=pool, state_indices=dev_i32(inp.state_indices),
              has_initial_state=dev_i32(inp.has_initial_state), write_final_to_pool=True,
              chunk_states_out=states)
    args = api.prefill_args(x, dt, A, B, C, 64, *md, **kw)
    ws = torch.empty(max(api.ssd_prefill_workspace_size(args), 256), dtype=torch.uint8,
                     device="cuda")
    api.ssd_prefill(x, dt, A, B, C, 64, *md, workspace=ws, **kw)
    torch.cuda.synchronize()
    y_eager, st_eager, pool_eager = y.clone(), states.clone(), pool.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            api.ssd_prefill(x, dt, A, B, C, 64, *md, workspace=ws, stream=s, **kw)
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(3):
        pool.copy_(pool0)
        y.zero_()
        states.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager)
        assert torch.equal(states, st_eager)
        assert torch.equal(pool, pool_eager)
        _ = (x.float() * 2).sum().item()       # unrelated eager work between replays
