"""Every output of the full-size workloads against the fp64 oracle.

The tiny fp32 prefill (1 x 256 tokens, 4 heads, head_dim 16, dstate 16, chunk 64), the
Mamba2-2.7B-like layer (4 x 2048 tokens, 80 heads, head_dim 64, dstate 128, chunk 256),
the Nemotron-H-like prefix-cache shard (16 varlen sequences resuming at unaligned points
from a 1024-slot pool, 48 heads, 4 groups), the speculative decode (256 live rows of a
512-row batch, 1 + 3 tokens, [2048, 48, 64, 128] pool) and the Mamba1 long-context scan
(8 x 16384 tokens, 5120 channels, 64 checkpoints) run once each through the C ABI, in the
kernels and launch shapes the benchmark times.  Then, one sequence (or every live row) at
a time, the oracle computes the same outputs and every element is compared: y, every
chunk-end state, every written pool slot (per output tensor, max |got - ref| <= 2e-2 max
|ref| for bf16 inputs, 1e-4 for fp32), with the checkpoint positions, padding rows and
untouched slots bit-exact.  The work of a chain or march workgroup depends on where it
runs (head -> XCD placement, chunk order, the hand-off form), so no sequence, head or
channel is left out."""
import numpy as np
import pytest

from gpu_helpers import TOL, check_prefill, oracle_prefill, run_decode, run_prefill
from selective_state_space_mamba2_amd.inputs import workload

pytestmark = pytest.mark.gpu


def _every_sequence(inp, got):
    """Oracle and comparison one sequence at a time (bounded host memory)."""
    worst = 0.0
    for r in range(inp.num_seqs):
        worst = max(worst, check_prefill(inp, got, oracle_prefill(inp, seqs=[r])))
    return worst


def _untouched_slots(inp, got):
    owned = set(int(v) for v in inp.state_indices)
    untouched = [s for s in range(inp.pool.shape[0]) if s not in owned]
    np.testing.assert_array_equal(got["pool"][untouched], inp.pool[untouched])


def test_every_output_tiny_fp32():
    inp = workload("tiny_fp32")
    got = run_prefill(inp)
    assert got["flag"] == 0
    assert len(got["metadata"][1]) == 4
    assert _every_sequence(inp, got) <= TOL["f32"]


def test_every_output_mamba2_2p7b_prefill():
    inp = workload("mamba2_2.7b_prefill")
    got = run_prefill(inp)
    assert got["flag"] == 0
    assert got["states"].shape[0] == 32
    _every_sequence(inp, got)


def test_every_output_nemotron_prefix_cache():
    inp = workload("nemotron_h_prefix_cache")
    got = run_prefill(inp)
    assert got["flag"] == 0
    # every first chunk is partial: the resume points are not multiples of the chunk size
    assert (np.asarray(inp.num_computed) % inp.chunk_size != 0).all()
    _every_sequence(inp, got)          # y, all chunk states, every written pool slot
    _untouched_slots(inp, got)


def test_every_output_decode_spec():
    from test_gpu_decode import _check
    inp = workload("decode_spec")
    got = run_decode(inp)
    assert got["flag"] == 0
    y_ref, writes = _check(inp, got)   # every live row, every written slot, padding rows
    assert len(y_ref) == inp.n_live and len(writes) == inp.n_live * inp.ntok


def test_every_output_mamba1_long_diag():
    inp = workload("mamba1_long_diag")
    got = run_prefill(inp)
    assert got["flag"] == 0
    assert got["states"].shape[0] == 64
    _every_sequence(inp, got)
