"""SSD_DEBUG: the distinct-slot precondition of the in-place pool updates, checked on the
device by an extra kernel each call launches first when the environment variable is set.

Two sequences (prefill) or two decode rows sharing a pool slot race on it; the check raises
SSD_DEVERR_DUPLICATE_SLOT.  With distinct slots it raises nothing and the results still
match the oracle; without SSD_DEBUG no check runs."""
import numpy as np
import pytest

from gpu_helpers import (TOL, assert_close, check_prefill, oracle_decode, oracle_prefill,
                         run_decode, run_prefill)
from selective_state_space_mamba2_amd import _abi
from selective_state_space_mamba2_amd.inputs import make_decode, make_prefill

pytestmark = pytest.mark.gpu

DUP = _abi.SSD_DEVERR_DUPLICATE_SLOT


def _decode_case():
    return make_decode(81, in_dtype="f32", B_pad=8, n_live=5, ntok=3, H=4, P=64, G=2, N=128,
                       pool_slots=32)


def test_decode_distinct_slots_pass_and_match(monkeypatch):
    monkeypatch.setenv("SSD_DEBUG", "1")
    d = _decode_case()
    got = run_decode(d)
    assert got["flag"] == 0
    y_ref, writes = oracle_decode(d)
    yh = got["y"].cpu().numpy()
    for r, yr in y_ref.items():
        assert_close(yh[r], yr, TOL["f32"], f"row {r}")
    for slot, st in writes.items():
        assert_close(got["pool"][slot], st, TOL["f32"], f"slot {slot}")


def test_decode_shared_slot_is_flagged(monkeypatch):
    d = _decode_case()
    d.state_indices[3, 2] = d.state_indices[1, 0]      # rows 1 and 3 both write one slot
    monkeypatch.setenv("SSD_DEBUG", "0")
    assert run_decode(d)["flag"] & DUP == 0            # checks off: not detected
    monkeypatch.setenv("SSD_DEBUG", "1")
    assert run_decode(d)["flag"] & DUP


def test_decode_padding_rows_may_share_the_null_slot(monkeypatch):
    monkeypatch.setenv("SSD_DEBUG", "1")
    d = _decode_case()
    assert (d.state_indices[d.n_live:] == d.null_block_id).all()
    assert run_decode(d)["flag"] == 0


def _prefill_case():
    return make_prefill(82, in_dtype="bf16", H=4, P=64, G=1, N=128, chunk_size=256,
                        lengths=[300, 90, 500], num_computed=[0, 7, 260], init="pool",
                        pool_slots=8)


def test_prefill_distinct_slots_pass_and_match(monkeypatch):
    monkeypatch.setenv("SSD_DEBUG", "1")
    inp = _prefill_case()
    got = run_prefill(inp)
    assert got["flag"] == 0
    check_prefill(inp, got, oracle_prefill(inp))


def test_prefill_shared_slot_is_flagged(monkeypatch):
    inp = _prefill_case()
    inp.state_indices[2] = inp.state_indices[0]
    monkeypatch.setenv("SSD_DEBUG", "1")
    assert run_prefill(inp)["flag"] & DUP
    monkeypatch.delenv("SSD_DEBUG")
    assert run_prefill(inp)["flag"] & DUP == 0


def test_prefill_all_cache_mode_overlapping_entries_are_flagged(monkeypatch):
    """Sequence 1's block entries overlap sequence 0's in the all cache mode."""
    from test_gpu_prefix_cache import _case, _lengths, _run
    cs, bs = 128, 256
    lengths, nc = _lengths(cs, bs)
    inp, table, lc, ls = _case(83, "bf16", 64, 128, cs, bs, lengths, nc)
    monkeypatch.setenv("SSD_DEBUG", "1")
    assert _run(inp, table, bs, lc, ls)["flag"] == 0
    table = table.copy()
    table[1, ls[1]] = table[0, 0]                     # sequence 0 writes block 0's entry
    assert _run(inp, table, bs, lc, ls)["flag"] & DUP
