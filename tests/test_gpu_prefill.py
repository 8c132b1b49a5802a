"""GPU parity of the chunked SSD prefill (scalar A per head) against the fp64 oracle.

Small cases run the oracle on every output element; the full-size workloads compare a
sample of sequences and heads the oracle can finish in seconds, plus properties that hold
at any size (finite outputs, untouched pool slots bit-identical)."""
import math

import numpy as np
import pytest

from gpu_helpers import (TOL, assert_close, check_prefill, oracle_prefill, pool_tol,
                         rounded_pool, run_prefill)
from oracle import transform_dt
from selective_state_space_mamba2_amd.inputs import make_prefill, workload

pytestmark = pytest.mark.gpu


def _case(seed, in_dtype, P, N, cs, lengths, nc, H=8, G=2, init="pool", slots=16, **kw):
    return make_prefill(seed, in_dtype=in_dtype, H=H, P=P, G=G, N=N, chunk_size=cs,
                        lengths=lengths, num_computed=nc, init=init, pool_slots=slots, **kw)


VARIANTS = [("bf16", 64, 128, 256), ("bf16", 64, 128, 128), ("bf16", 64, 128, 64),
            ("bf16", 16, 16, 64), ("f32", 16, 16, 64), ("f32", 64, 128, 64),
            ("bf16", 16, 16, 256), ("f32", 16, 16, 256), ("f32", 64, 128, 256),
            # the rest of the minimum instantiation set: head_dim 16 with dstate 128, head_dim
            # 64 with dstate 16 (chunked kernels), head_dim 1 (the sequential scan)
            ("bf16", 16, 128, 64), ("bf16", 16, 128, 256), ("bf16", 64, 16, 64),
            ("bf16", 64, 16, 256), ("f32", 16, 128, 64), ("f32", 16, 128, 256),
            ("f32", 64, 16, 64), ("f32", 64, 16, 256),
            ("bf16", 1, 16, 64), ("bf16", 1, 16, 256), ("bf16", 1, 128, 64),
            ("bf16", 1, 128, 256), ("f32", 1, 16, 64), ("f32", 1, 16, 256),
            ("f32", 1, 128, 64), ("f32", 1, 128, 256)]


@pytest.mark.parametrize("dtype,P,N,cs", VARIANTS)
def test_ragged_varlen_with_pool(dtype, P, N, cs):
    """Three sequences spanning several chunks with unaligned resume points and a ragged
    tail; sequences 0 and 2 start from pool states, sequence 1 from zero (both initial-state
    paths in one call); final states go back to the pool."""
    inp = _case(100 + cs + P, dtype, P, N, cs, [3 * cs + 17, 5, 2 * cs - 1],
                [0, cs + 3, 7])
    inp.has_initial_state[1] = 0
    got = run_prefill(inp)
    assert got["flag"] == 0
    check_prefill(inp, got, oracle_prefill(inp))
    # slots not owned by any sequence are bit-identical
    owned = set(int(v) for v in inp.state_indices)
    for s in range(inp.pool.shape[0]):
        if s not in owned:
            np.testing.assert_array_equal(got["pool"][s], inp.pool[s])


def test_tiny_fp32_workload():
    inp = workload("tiny_fp32")
    got = run_prefill(inp)
    assert got["flag"] == 0
    assert len(got["metadata"][1]) == 4
    check_prefill(inp, got, oracle_prefill(inp))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_initial_states_without_pool(dtype):
    inp = _case(7, dtype, 64, 128, 64, [200, 64, 1], [0, 0, 63], init="none")
    got = run_prefill(inp)
    check_prefill(inp, got, oracle_prefill(inp))


def test_partial_and_single_token_chunks():
    """Chunks of length 1 and cs-1 at both ends of sequences, and a one-token sequence."""
    cs = 256
    inp = _case(8, "bf16", 64, 128, cs, [1, cs - 1, cs + 1, 2, 1], [cs - 1, 1, 0, cs - 1, 5])
    got = run_prefill(inp)
    lens = np.diff(got["metadata"][0])
    assert lens.min() == 1 and (lens == cs - 1).any()
    check_prefill(inp, got, oracle_prefill(inp))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_long_memory_and_zero_decay(dtype):
    """Small |A| (state carried across many chunks) and A = 0 (a plain prefix sum)."""
    inp = _case(9, dtype, 64, 128, 64, [700, 300], [0, 10], A_range=(1e-3, 1e-2))
    check_prefill(inp, run_prefill(inp), oracle_prefill(inp))
    inp0 = _case(10, dtype, 64, 128, 64, [500], [0], A_zero=True, init="none")
    check_prefill(inp0, run_prefill(inp0), oracle_prefill(inp0))


@pytest.mark.parametrize("dtype,N", [("bf16", 128), ("f32", 16)])
def test_head_dim_one(dtype, N):
    """head_dim 1 (the sequential scan with A per head): heads whose group spans several
    workgroups (80 heads, 2 groups), long memory and A = 0, softplus with bias and limit."""
    inp = _case(21, dtype, 1, N, 64, [300, 1, 130], [0, 63, 5], H=80, G=2, slots=8,
                A_range=(1e-3, 1e-2))
    check_prefill(inp, run_prefill(inp), oracle_prefill(inp))
    inp0 = _case(22, dtype, 1, N, 256, [500], [0], H=8, G=4, A_zero=True, init="none")
    check_prefill(inp0, run_prefill(inp0), oracle_prefill(inp0))
    bias = np.linspace(-1.5, 0.5, 80).astype(np.float32).astype(np.float64)
    got = run_prefill(inp, dt_bias=bias, softplus=True, dt_limit=(0.01, 0.5), write_final=False)
    ref = oracle_prefill(inp, dt_bias=bias, softplus=True, dt_limit=(0.01, 0.5))
    check_prefill(inp, got, ref, check_pool=False)


def test_dt_zero_keeps_the_state():
    inp = _case(11, "bf16", 64, 128, 256, [300, 40], [0, 0], dt_zero=True)
    got = run_prefill(inp)
    check_prefill(inp, got, oracle_prefill(inp))
    for r in range(2):   # dt = 0: the final state is the initial one, exactly
        s = int(inp.state_indices[r])
        np.testing.assert_array_equal(got["pool"][s], inp.pool[s])


@pytest.mark.parametrize("dtype,cs", [("bf16", 256), ("f32", 64)])
def test_dt_bias_softplus_and_limit(dtype, cs):
    inp = _case(12, dtype, 64, 128, cs, [cs + 40, 90], [0, 3])
    rng = np.random.default_rng(5)
    bias = rng.normal(-1.0, 0.5, size=inp.H).astype(np.float32).astype(np.float64)
    for limit in [(0.0, math.inf), (0.05, 0.4)]:
        got = run_prefill(inp, dt_bias=bias, softplus=True, dt_limit=limit, write_final=False)
        ref = oracle_prefill(inp, dt_bias=bias, softplus=True, dt_limit=limit)
        check_prefill(inp, got, ref, check_pool=False)


def test_strided_projection_views_and_no_D():
    inp = _case(13, "bf16", 64, 128, 256, [400, 130], [5, 0])
    got = run_prefill(inp, views=True, use_D=False)
    check_prefill(inp, got, oracle_prefill(inp, use_D=False))


def test_without_chunk_state_output_uses_workspace():
    inp = _case(14, "bf16", 64, 128, 128, [333, 200], [0, 50])
    got = run_prefill(inp, want_states=False)
    check_prefill(inp, got, oracle_prefill(inp))


def test_long_chain_without_state_output():
    """Seven chunks of one sequence with no chunk-state output: the chain kernel hands the
    state down through its two-deep workspace ring, so entries are overwritten while the
    sequence runs; a second sequence resumes mid-chunk."""
    inp = _case(16, "bf16", 64, 128, 128, [7 * 128 - 5, 300], [0, 77])
    got = run_prefill(inp, want_states=False)
    assert got["flag"] == 0
    check_prefill(inp, got, oracle_prefill(inp))


def test_many_short_sequences_take_chunks_in_index_order():
    """More sequences than the prep kernel orders (1100 > 1024): the chain kernel then
    takes chunks in index order, which also dispatches every predecessor first."""
    rng = np.random.default_rng(17)
    lengths = [int(v) for v in rng.integers(1, 4, size=1100)]
    lengths[5] = 300                                  # one multi-chunk sequence in the mix
    inp = _case(17, "bf16", 64, 128, 128, lengths, [0] * 1100, H=4, G=1, slots=1200)
    got = run_prefill(inp)
    assert got["flag"] == 0
    check_prefill(inp, got, oracle_prefill(inp, seqs=[0, 5, 6, 700, 1099]))


@pytest.mark.parametrize("pool", ["bf16", "f16"])
@pytest.mark.parametrize("dtype,P,N,cs", [("bf16", 64, 128, 256), ("bf16", 64, 128, 64),
                                          ("f32", 64, 128, 64), ("f32", 64, 128, 256)])
def test_2byte_state_pool(pool, dtype, P, N, cs):
    """Initial states gathered from, and final states written to, a bf16 or fp16 pool (chain
    and march kernels); y and the fp32 chunk states keep the input dtype's tolerance, the
    written pool slots the pool type's where that is looser, untouched slots stay
    bit-identical."""
    inp = rounded_pool(_case(36, dtype, P, N, cs, [2 * cs + 40, cs - 3, 70], [0, 5, cs - 1]),
                       pool)
    got = run_prefill(inp)
    assert got["flag"] == 0
    check_prefill(inp, got, oracle_prefill(inp), pool_tol=pool_tol(inp))
    owned = set(int(v) for v in inp.state_indices)
    untouched = [s for s in range(inp.pool.shape[0]) if s not in owned]
    np.testing.assert_array_equal(got["pool"][untouched], inp.pool[untouched])


@pytest.mark.parametrize("dtype,P,N,cs", [("bf16", 64, 128, 256), ("f32", 16, 16, 64)])
def test_graph_capture_and_replay(dtype, P, N, cs):
    """The prefill (chain or march kernels) captured in a HIP graph, replayed several times
    with eager work in between, gives the eager call's y, chunk states and pool on every
    replay (the workspace's flags and counters are reset by the kernels, not by a memset)."""
    import torch
    from gpu_helpers import dev_f32, dev_i32, dev_token, prefill_metadata
    from selective_state_space_mamba2_amd import api
    inp = _case(35, dtype, P, N, cs, [3 * cs + 17, cs - 5, 2 * cs], [0, 11, cs + 3])
    cuc, sidx, last = prefill_metadata(inp)
    x, dt, B, C = (dev_token(inp, n) for n in ("x", "dt", "B", "C"))
    A, D = dev_f32(inp.A), dev_f32(inp.D)
    md = [dev_i32(inp.cu_seqlens), dev_i32(cuc), dev_i32(sidx), dev_i32(last)]
    pool0 = torch.from_numpy(inp.pool).cuda()
    pool = pool0.clone()
    y = torch.zeros_like(x)
    states = torch.zeros(len(sidx), inp.H, P, N, device="cuda")
    kw = dict(y=y, D=D, state_pool=pool, state_indices=dev_i32(inp.state_indices),
              has_initial_state=dev_i32(inp.has_initial_state), write_final_to_pool=True,
              chunk_states_out=states)
    args = api.prefill_args(x, dt, A, B, C, cs, *md, **kw)
    ws = torch.empty(max(api.ssd_prefill_workspace_size(args), 256), dtype=torch.uint8,
                     device="cuda")
    api.ssd_prefill(x, dt, A, B, C, cs, *md, workspace=ws, **kw)
    torch.cuda.synchronize()
    y_eager, st_eager, pool_eager = y.clone(), states.clone(), pool.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            api.ssd_prefill(x, dt, A, B, C, cs, *md, workspace=ws, stream=s, **kw)
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(3):
        pool.copy_(pool0)
        y.zero_()
        states.zero_()
        ws.fill_(255)                          # stale flags and counters from elsewhere
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager)
        assert torch.equal(states, st_eager)
        assert torch.equal(pool, pool_eager)
        _ = (x.float() * 2).sum().item()       # unrelated eager work between replays


@pytest.mark.parametrize("dtype,cs", [("bf16", 256), ("f32", 64)])
def test_per_step_outputs(dtype, cs):
    """The within-chunk cumsum of delta*A, C.B^T per chunk and group, and each chunk's
    own state from zero, against their definitions evaluated from the same inputs."""
    inp = _case(15, dtype, 64, 128, cs, [cs + 70, 33], [0, 9], init="none")
    got = run_prefill(inp, debug=True)
    cuc, sidx, _ = got["metadata"]
    delta = transform_dt(inp.values("dt"))
    Bv, Cv = inp.values("B"), inp.values("C")
    tol = TOL[dtype]
    exp_cum = np.zeros((inp.H, inp.T))
    for k in range(len(sidx)):
        a, b = cuc[k], cuc[k + 1]
        exp_cum[:, a:b] = np.cumsum(delta[a:b] * inp.A[None, :], axis=0).T
        cb = np.einsum("lgn,sgn->gls", Cv[a:b], Bv[a:b])
        L = b - a
        mask = np.tril(np.ones((L, L), dtype=bool))
        for g in range(inp.G):
            assert_close(got["cb_out"][k, g, :L, :L][mask], cb[g][mask], 1e-5, f"CB chunk {k}")
        # the chunk's own state: the oracle run over the chunk alone from a zero state
        r = sidx[k]
        loc = oracle_prefill_chunk(inp, a, b)
        assert_close(got["chunk_local_states_out"][k], loc, tol, f"local state chunk {k}")
    assert_close(got["dA_cumsum_out"], exp_cum, 1e-5, "dA cumsum")


def oracle_prefill_chunk(inp, a, b):
    from oracle import scan_prefill
    o = scan_prefill(inp.values("x")[a:b], inp.values("dt")[a:b], inp.A, inp.values("B")[a:b],
                     inp.values("C")[a:b], inp.D, [0, b - a], chunk_size=b - a + 1)
    return o["final_states"][0]


def test_out_of_range_slot_raises_the_device_flag():
    inp = _case(16, "bf16", 64, 128, 256, [100, 50], [0, 0])
    bad = inp.state_indices.copy()
    inp.state_indices[1] = inp.pool.shape[0]          # outside [0, num_slots)
    got = run_prefill(inp)
    assert got["flag"] & 2
    # the sequence with the bad slot ran from a zero state and wrote no slot
    inp2 = _case(16, "bf16", 64, 128, 256, [100, 50], [0, 0])
    np.testing.assert_array_equal(got["pool"][int(bad[1])], inp2.pool[int(bad[1])])
    inp.has_initial_state[1] = 0
    ref = oracle_prefill(inp, seqs=[0, 1])
    check_prefill(inp, got, {0: ref[0]})
    assert_close(got["y"][100:150], ref[1]["y"], TOL["bf16"], "y of the flagged sequence")


def test_default_error_word_keeps_device_errors():
    """A call given no device_error_flag reports into the GPU's persistent error word,
    which check_device_errors turns into an exception (and clears)."""
    from gpu_helpers import dev_f32, dev_i32, dev_token, prefill_metadata
    from selective_state_space_mamba2_amd import api
    inp = _case(16, "bf16", 64, 128, 256, [100, 50], [0, 0])
    inp.state_indices[1] = inp.pool.shape[0]          # outside [0, num_slots)
    api.ssd_device_errors()                           # start from a clear word
    cuc, sidx, last = prefill_metadata(inp)
    import torch
    pool = torch.from_numpy(inp.pool).cuda()
    api.ssd_prefill(*(dev_token(inp, n) for n in ("x", "dt")), dev_f32(inp.A),
                    *(dev_token(inp, n) for n in ("B", "C")), inp.chunk_size,
                    dev_i32(inp.cu_seqlens), dev_i32(cuc), dev_i32(sidx), dev_i32(last),
                    state_pool=pool, state_indices=dev_i32(inp.state_indices),
                    has_initial_state=dev_i32(inp.has_initial_state), write_final_to_pool=True)
    with pytest.raises(RuntimeError, match="SLOT_RANGE"):
        api.check_device_errors()
    assert api.ssd_device_errors() == 0               # cleared by the check


# ----------------------------------------------------------------------------------------
# full-size workloads (sampled against the oracle)
# ----------------------------------------------------------------------------------------
def test_full_mamba2_2p7b_prefill():
    inp = workload("mamba2_2.7b_prefill")
    got = run_prefill(inp)
    assert got["flag"] == 0 and np.isfinite(got["y"]).all()
    heads = [0, 41, 79]
    check_prefill(inp, got, oracle_prefill(inp, seqs=[1], heads=heads), heads=heads)


def test_full_nemotron_prefix_cache():
    inp = workload("nemotron_h_prefix_cache")
    got = run_prefill(inp)
    assert got["flag"] == 0 and np.isfinite(got["y"]).all()
    lengths = np.diff(inp.cu_seqlens)
    seqs = [int(np.argmin(lengths)), int(np.argmax(lengths))]
    heads = [3, 12 + 7, 24 + 0, 36 + 11]
    check_prefill(inp, got, oracle_prefill(inp, seqs=seqs, heads=heads), heads=heads)
    owned = set(int(v) for v in inp.state_indices)
    untouched = [s for s in range(inp.pool.shape[0]) if s not in owned]
    np.testing.assert_array_equal(got["pool"][untouched], inp.pool[untouched])



def test_two_streams_at_once():
    """Two independent chain-kernel prefills issued on two streams at the same time, several
    times over: each gives exactly the outputs it gives alone and raises no device error
    (the hand-off assumes that a predecessor and its successor, whose workgroup ids are
    equal mod 8, run on one XCD also while another launch shares the device)."""
    import torch
    from gpu_helpers import dev_f32, dev_i32, dev_token, prefill_metadata
    from selective_state_space_mamba2_amd import api
    calls = []
    for seed in (37, 38):
        inp = _case(seed, "bf16", 64, 128, 256, [1500, 900, 2300, 400], [0, 300, 77, 255],
                    H=16, G=2)
        cuc, sidx, last = prefill_metadata(inp)
        x, dt, B, C = (dev_token(inp, n) for n in ("x", "dt", "B", "C"))
        md = [dev_i32(inp.cu_seqlens), dev_i32(cuc), dev_i32(sidx), dev_i32(last)]
        pool0 = torch.from_numpy(inp.pool).cuda()
        out = dict(y=torch.zeros_like(x), pool=pool0.clone(),
                   states=torch.zeros(len(sidx), inp.H, 64, 128, device="cuda"),
                   flag=torch.zeros(1, dtype=torch.int32, device="cuda"))
        kw = dict(y=out["y"], D=dev_f32(inp.D), state_pool=out["pool"],
                  state_indices=dev_i32(inp.state_indices),
                  has_initial_state=dev_i32(inp.has_initial_state), write_final_to_pool=True,
                  chunk_states_out=out["states"], device_error_flag=out["flag"])
        a = api.prefill_args(x, dt, dev_f32(inp.A), B, C, 256, *md, **kw)
        ws = torch.empty(max(api.ssd_prefill_workspace_size(a), 256), dtype=torch.uint8,
                         device="cuda")
        run = (lambda st, x=x, dt=dt, A=dev_f32(inp.A), B=B, C=C, md=md, kw=kw, ws=ws:
               api.ssd_prefill(x, dt, A, B, C, 256, *md, workspace=ws, stream=st, **kw))
        calls.append((run, out, pool0))
    main = torch.cuda.current_stream()
    ref = []
    for run, out, pool0 in calls:
        run(main)
        torch.cuda.synchronize()
        assert int(out["flag"].item()) == 0
        ref.append({k: out[k].clone() for k in ("y", "states", "pool")})
    side = torch.cuda.Stream()
    for _ in range(4):
        for run, out, pool0 in calls:
            out["pool"].copy_(pool0)
            out["y"].zero_()
            out["states"].zero_()
        side.wait_stream(main)
        calls[0][0](main)
        calls[1][0](side)
        torch.cuda.synchronize()
        for (run, out, pool0), r in zip(calls, ref):
            assert int(out["flag"].item()) == 0
            assert torch.equal(out["y"], r["y"])
            assert torch.equal(out["states"], r["states"])
            assert torch.equal(out["pool"], r["pool"])


def test_argument_struct_keeps_its_tensors_alive():
    """An argument struct built from temporaries (every token, metadata and index tensor
    dropped by the caller) still runs correctly after a garbage collection and a burst of
    allocations that would reuse freed blocks: the struct holds the tensors it points into."""
    import ctypes
    import gc

    from gpu_helpers import dev_f32, dev_i32, dev_token, prefill_metadata, torch
    from selective_state_space_mamba2_amd import api
    from selective_state_space_mamba2_amd._abi import check, lib
    t = torch()
    inp = _case(71, "bf16", 64, 128, 256, [600, 257, 90], [0, 40, 255])
    cuc, sidx, last = prefill_metadata(inp)
    y = t.full((inp.T, inp.H, inp.P), float("nan"), dtype=t.bfloat16, device="cuda")
    pool = t.from_numpy(inp.pool).cuda()
    states = t.full((len(sidx), inp.H, inp.P, inp.N), float("nan"), device="cuda")
    flag = t.zeros(1, dtype=t.int32, device="cuda")

    def build():
        return api.prefill_args(
            dev_token(inp, "x"), dev_token(inp, "dt"), dev_f32(inp.A), dev_token(inp, "B"),
            dev_token(inp, "C"), inp.chunk_size, dev_i32(inp.cu_seqlens), dev_i32(cuc),
            dev_i32(sidx), dev_i32(last), y, D=dev_f32(inp.D), state_pool=pool,
            state_indices=dev_i32(inp.state_indices),
            has_initial_state=dev_i32(inp.has_initial_state), write_final_to_pool=True,
            chunk_states_out=states, device_error_flag=flag)

    a = build()
    gc.collect()
    junk = [t.full((n,), -7, dtype=t.int32, device="cuda") for n in (1, 4, 17, 256, 4096) * 8]
    ws = t.empty(max(api.ssd_prefill_workspace_size(a), 256), dtype=t.uint8, device="cuda")
    check("ssd_prefill", lib().ssd_prefill(ctypes.byref(a), ws.data_ptr(), ws.numel(),
                                           t.cuda.current_stream().cuda_stream))
    t.cuda.synchronize()
    assert int(flag.item()) == 0
    got = dict(y=y.float().cpu().numpy().astype(np.float64), metadata=(cuc, sidx, last),
               states=states.cpu().numpy().astype(np.float64), pool=pool.cpu().numpy())
    check_prefill(inp, got, oracle_prefill(inp))
    del junk
