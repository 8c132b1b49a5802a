"""GPU parity of the all cache mode: prefix caching with one pool entry per cache block.

The prefill reads a sequence's initial state from its block_idx_last_computed entry, writes
the state at every block end to that block's entry and the final state to the
block_idx_last_scheduled entry; the decode reads the last-computed entry and writes the
last-scheduled one.  Every run is compared with the fp64 oracle on the same seeded inputs:
y and the chunk states at the input dtype's tolerance, every written pool entry at the
pool dtype's, and every other slot bit-identical.
"""
import numpy as np
import pytest

from gpu_helpers import (TOL, _dev_pool, _vals, assert_close, dev_f32, dev_i32, dev_token,
                         host64, pool_tol, prefill_metadata, rounded_pool, torch)
from oracle import block_indices, scan_decode, scan_prefill
from selective_state_space_mamba2_amd import _abi, api
from selective_state_space_mamba2_amd.inputs import make_decode, make_prefill

pytestmark = pytest.mark.gpu


def _block_table(seed, rows, max_blocks, slots):
    """Distinct pool slots in [1, slots) for every (row, block) entry."""
    rng = np.random.default_rng(seed)
    assert rows * max_blocks < slots
    return (rng.permutation(slots - 1)[:rows * max_blocks] + 1).reshape(rows, max_blocks).astype(np.int32)


def _columns(nc, lengths, bs):
    """The caller's block columns; they agree with the oracle's reading of the names."""
    nc, L = np.asarray(nc), np.asarray(lengths)
    lc = np.where(nc > 0, (nc - 1) // bs, -1).astype(np.int32)
    ls = ((nc + L - 1) // bs).astype(np.int32)
    _, lc_o, ls_o = block_indices(nc, L, bs)
    np.testing.assert_array_equal(lc, lc_o)
    np.testing.assert_array_equal(ls, ls_o)
    return lc, ls


def _case(seed, dtype, P, N, cs, bs, lengths, nc, H=4, G=2, max_blocks=4, a_kind="scalar"):
    S = len(lengths)
    inp = make_prefill(seed, in_dtype=dtype, H=H, P=P, G=G, N=N, chunk_size=cs,
                       lengths=lengths, num_computed=nc, init="pool",
                       pool_slots=S * max_blocks + 1, a_kind=a_kind)
    table = _block_table(seed + 1, S, max_blocks, inp.pool.shape[0])
    lc, ls = _columns(nc, lengths, bs)
    assert ls.max() < max_blocks
    return inp, table, lc, ls


def _run(inp, table, bs, lc, ls, *, write_final=True, want_states=True,
         nc_dev=None):
    t = torch()
    cuc, sidx, last = prefill_metadata(inp)
    x, dt, B, C = (dev_token(inp, n) for n in ("x", "dt", "B", "C"))
    y = t.full_like(x, float("nan"))
    pool = _dev_pool(inp)
    has_init = (inp.num_computed > 0).astype(np.int32)
    states = (t.full((len(sidx), inp.H, inp.P, inp.N), float("nan"), device="cuda")
              if want_states else None)
    flag = t.zeros(1, dtype=t.int32, device="cuda")
    nc = inp.num_computed if nc_dev is None else nc_dev
    api.ssd_prefill(
        x, dt, dev_f32(inp.A), B, C, inp.chunk_size, dev_i32(inp.cu_seqlens), dev_i32(cuc),
        dev_i32(sidx), dev_i32(last), y=y, D=dev_f32(inp.D), state_pool=pool,
        state_indices=dev_i32(table), has_initial_state=dev_i32(has_init),
        write_final_to_pool=write_final, chunk_states_out=states, device_error_flag=flag,
        block_size=bs, num_computed=dev_i32(nc), block_idx_last_computed=dev_i32(lc),
        block_idx_last_scheduled=dev_i32(ls))
    t.cuda.synchronize()
    return dict(y=host64(y), pool=pool.float().cpu().numpy(), flag=int(flag.item()),
                states=None if states is None else states.cpu().numpy().astype(np.float64),
                sidx=sidx)


def _expected(inp, table, bs, lc, ls, write_final=True):
    """The oracle per sequence, and the pool entries the call must write."""
    cu = inp.cu_seqlens
    refs, writes = {}, {}
    for r in range(len(cu) - 1):
        t0, t1 = int(cu[r]), int(cu[r + 1])
        rows = slice(t0, t1)
        nc = int(inp.num_computed[r])
        h0 = inp.pool[table[r, lc[r]]].astype(np.float64) if nc > 0 else None
        o = scan_prefill(_vals(inp, "x", rows), _vals(inp, "dt", rows), inp.A,
                         _vals(inp, "B", rows), _vals(inp, "C", rows), inp.D, [0, t1 - t0],
                         inp.chunk_size, num_computed=[nc], initial_states=[h0],
                         block_size=bs)
        refs[r] = o
        for _, col, h in o["block_states"]:
            writes[int(table[r, col])] = h
        if write_final:
            writes[int(table[r, ls[r]])] = o["final_states"][0]
    return refs, writes


def _check(inp, got, refs, writes, entry_tol):
    tol = TOL[inp.in_dtype]
    assert got["flag"] == 0
    for r, o in refs.items():
        t0, t1 = int(inp.cu_seqlens[r]), int(inp.cu_seqlens[r + 1])
        assert_close(got["y"][t0:t1], o["y"], tol, f"y seq {r}")
        if got["states"] is not None:
            ks = np.flatnonzero(got["sidx"] == r)
            assert_close(got["states"][ks], o["boundary_states"], tol, f"chunk states seq {r}")
    for slot, h in writes.items():
        assert_close(got["pool"][slot], h, entry_tol, f"pool slot {slot}")
    untouched = [s for s in range(inp.pool.shape[0]) if s not in writes]
    np.testing.assert_array_equal(got["pool"][untouched], inp.pool[untouched])


# (dtype, P, N, cs, bs): chain kernel shapes (bf16, P = 64) and march kernel shapes
SHAPES = [("bf16", 64, 128, 128, 256), ("bf16", 64, 128, 256, 256),
          ("f32", 16, 16, 64, 128), ("bf16", 64, 128, 64, 192)]


def _lengths(cs, bs):
    """Sequences that resume at 0, mid-block, at a block end and one token before one, one
    of them ending exactly on a block end."""
    nc = [0, bs // 2 - 7, bs, 2 * bs - 1]
    lengths = [2 * bs + cs + 13, 2 * bs - nc[1], cs // 2 + 1, 45]
    return lengths, nc


@pytest.mark.parametrize("dtype,P,N,cs,bs", SHAPES)
@pytest.mark.parametrize("write_final", [True, False])
def test_prefill_writes_every_block_entry(dtype, P, N, cs, bs, write_final):
    lengths, nc = _lengths(cs, bs)
    inp, table, lc, ls = _case(51, dtype, P, N, cs, bs, lengths, nc)
    got = _run(inp, table, bs, lc, ls, write_final=write_final)
    refs, writes = _expected(inp, table, bs, lc, ls, write_final)
    _check(inp, got, refs, writes, TOL[dtype])


@pytest.mark.parametrize("H", [200, 5120])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("write_final", [True, False])
def test_prefill_diag_writes_every_block_entry(dtype, write_final, H):
    """The Mamba1 scan (diagonal A [H, 16]; 200 channels leave a ragged last workgroup, 5120
    run the grid of 64- and 32-channel workgroups) in the all cache mode: y, the chunk
    states, every block-end entry and the final entry."""
    cs, bs = 64, 128
    lengths, nc = _lengths(cs, bs)
    inp, table, lc, ls = _case(55, dtype, 1, 16, cs, bs, lengths, nc, H=H, G=1,
                               a_kind="diag")
    got = _run(inp, table, bs, lc, ls, write_final=write_final)
    refs, writes = _expected(inp, table, bs, lc, ls, write_final)
    assert any(len(o["block_states"]) for o in refs.values())
    _check(inp, got, refs, writes, TOL[dtype])


@pytest.mark.parametrize("pool", ["bf16", "f16"])
def test_prefill_diag_2byte_pool(pool):
    """The same through a bf16 or fp16 pool (entries at the looser of the input's and the
    pool type's tolerance)."""
    cs, bs = 64, 192
    lengths, nc = _lengths(cs, bs)
    inp, table, lc, ls = _case(56, "bf16", 1, 16, cs, bs, lengths, nc, H=72, G=1,
                               a_kind="diag")
    rounded_pool(inp, pool)
    got = _run(inp, table, bs, lc, ls)
    refs, writes = _expected(inp, table, bs, lc, ls)
    _check(inp, got, refs, writes, pool_tol(inp))


@pytest.mark.parametrize("pool", ["bf16", "f16"])
@pytest.mark.parametrize("dtype,P,N,cs,bs", [SHAPES[0], SHAPES[2]])
def test_prefill_2byte_pool_and_no_chunk_state_output(dtype, P, N, cs, bs, pool):
    """A bf16 or fp16 pool (entries at the looser of the input's and the pool type's
    tolerance) and no chunk_states_out (the chain kernel hands states over through its
    workspace ring)."""
    lengths, nc = _lengths(cs, bs)
    inp, table, lc, ls = _case(52, dtype, P, N, cs, bs, lengths, nc)
    rounded_pool(inp, pool)
    got = _run(inp, table, bs, lc, ls, want_states=False)
    refs, writes = _expected(inp, table, bs, lc, ls)
    _check(inp, got, refs, writes, pool_tol(inp))


def test_prefill_resumes_from_its_own_entries():
    """Two calls: the first caches a sequence's blocks, the second resumes from the entry the
    first left (a partial block) and must give the one-shot result."""
    cs, bs, T = 128, 256, 900
    whole = make_prefill(53, in_dtype="bf16", H=4, P=64, G=1, N=128, chunk_size=cs,
                         lengths=[T], init="pool", pool_slots=9)
    table = _block_table(54, 1, 8, 9)
    one = _run(whole, table, bs, *_columns([0], [T], bs))
    cut = 333
    parts = []
    for lo, hi in ((0, cut), (cut, T)):
        p = make_prefill(53, in_dtype="bf16", H=4, P=64, G=1, N=128, chunk_size=cs,
                         lengths=[hi - lo], num_computed=[lo], init="pool", pool_slots=9)
        for name in ("x", "dt", "B", "C"):
            setattr(p, name, getattr(whole, name)[lo:hi])
        p.A, p.D = whole.A, whole.D
        p.pool = whole.pool if lo == 0 else parts[-1]["pool"]
        parts.append(_run(p, table, bs, *_columns([lo], [hi - lo], bs)))
    assert one["flag"] == 0 and parts[0]["flag"] == 0 and parts[1]["flag"] == 0
    y2 = np.concatenate([parts[0]["y"], parts[1]["y"]])
    assert_close(y2, one["y"], TOL["bf16"], "y resumed")
    assert_close(parts[1]["pool"], one["pool"], TOL["bf16"], "pool resumed")


def test_prefill_flags_inconsistent_columns():
    """A num_computed other than the one the chunks were built with puts a block end inside
    a chunk (SSD_DEVERR_CHUNK_RANGE); a last-scheduled column past the row raises
    SSD_DEVERR_SLOT_RANGE and skips that write."""
    cs, bs = 128, 256
    lengths, nc = _lengths(cs, bs)
    inp, table, lc, ls = _case(55, "bf16", 64, 128, cs, bs, lengths, nc)
    got = _run(inp, table, bs, lc, ls, nc_dev=np.asarray(nc) + np.array([17, 0, 0, 0]))
    assert got["flag"] & _abi.SSD_DEVERR_CHUNK_RANGE
    bad = ls.copy()
    bad[2] = table.shape[1]
    got = _run(inp, table, bs, lc, bad)
    assert got["flag"] == _abi.SSD_DEVERR_SLOT_RANGE
    refs, writes = _expected(inp, table, bs, lc, ls)
    del writes[int(table[2, ls[2]])]
    for slot, h in writes.items():
        assert_close(got["pool"][slot], h, TOL["bf16"], f"pool slot {slot}")
    np.testing.assert_array_equal(got["pool"][table[2, ls[2]]], inp.pool[table[2, ls[2]]])


@pytest.mark.parametrize("kind", ["scalar", "diag"])
@pytest.mark.parametrize("pool_dtype", ["f32", "bf16", "f16"])
def test_decode_reads_last_computed_writes_last_scheduled(kind, pool_dtype):
    t = torch()
    if kind == "scalar":
        inp = make_decode(56, in_dtype="bf16", B_pad=12, n_live=9, ntok=1, H=8, P=64, G=2,
                          N=128, pool_slots=64)
    else:
        inp = make_decode(57, in_dtype="bf16", B_pad=12, n_live=9, ntok=1, H=200, P=1, G=1,
                          N=16, pool_slots=64, a_kind="diag")
    if pool_dtype != "f32":
        rounded_pool(inp, pool_dtype)
    rng = np.random.default_rng(58)
    table = _block_table(59, 12, 3, 64)
    table[9:] = inp.null_block_id                          # padding rows
    lc = rng.integers(0, 3, size=12).astype(np.int32)
    ls = np.minimum(lc + rng.integers(0, 2, size=12), 2).astype(np.int32)
    x, dt, B, C = (dev_token(inp, n) for n in ("x", "dt", "B", "C"))
    y = t.full_like(x, 7.0)
    pool = _dev_pool(inp)
    flag = t.zeros(1, dtype=t.int32, device="cuda")
    api.ssd_state_update(x, dt, dev_f32(inp.A), B, C, pool, dev_i32(table), y=y,
                         null_block_id=inp.null_block_id, D=dev_f32(inp.D),
                         device_error_flag=flag, block_idx_last_computed=dev_i32(lc),
                         block_idx_last_scheduled=dev_i32(ls))
    t.cuda.synchronize()
    assert int(flag.item()) == 0
    y_ref, writes = scan_decode(inp.pool, table, None, inp.values("x"), inp.values("dt"),
                                inp.A, inp.values("B"), inp.values("C"), inp.D,
                                inp.null_block_id, block_idx_last_computed=lc,
                                block_idx_last_scheduled=ls)
    assert set(y_ref) == set(range(9))
    yh = host64(y)
    for r, yr in y_ref.items():
        assert_close(yh[r], yr, TOL["bf16"], f"y row {r}")
    assert np.all(yh[9:] == 7.0)                          # padding rows untouched
    got = pool.float().cpu().numpy()
    for slot, h in writes.items():
        assert_close(got[slot], h, TOL[pool_dtype], f"slot {slot}")
    untouched = [s for s in range(inp.pool.shape[0]) if s not in writes]
    np.testing.assert_array_equal(got[untouched], inp.pool[untouched])
