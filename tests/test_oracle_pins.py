"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test checks the oracle against something independent: a hand-derived worked example,
a brute-force unrolled quadratic form written separately here, closed forms (A = 0, the
time-invariant geometric series, scipy's IIR filter), invariants (dt = 0, chunk-split
invariance) and the chunk-metadata examples printed or derived from the pages.  Each is
chosen so a plausible slip in the oracle (a dropped term, a sign, a swapped B/C, a wrong
head->group index, an off-by-one in the checkpoint positions) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.signal

from oracle import block_indices, chunk_metadata, scan_decode, scan_prefill, transform_dt

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(seed, T, H, P, G, N, S=1, init=False, a_scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H, P))
    dt = np.logaddexp(0.0, rng.standard_normal((T, H)) - 1.0)
    A = -np.exp(rng.uniform(0.0, np.log(4.0), size=H)) * a_scale
    B = rng.standard_normal((T, G, N))
    C = rng.standard_normal((T, G, N))
    D = rng.standard_normal(H)
    cuts = np.sort(rng.choice(np.arange(1, T), size=S - 1, replace=False)) if S > 1 else []
    cu = np.array([0, *cuts, T])
    h0 = [rng.standard_normal((H, P, N)) * 0.5 for _ in range(S)] if init else None
    return x, dt, A, B, C, D, cu, h0


def _bruteforce_y(x, delta, A, B, C, D, cu, h0):
    """Unrolled closed form, a double loop written independently of the oracle:
    y_t = exp(sum_{r<=t} d_r A) (h0 C_t) + sum_{s<=t} exp(sum_{s<r<=t} d_r A) d_s (C_t.B_s) x_s
          + D x_t, per head, with the group of head h being h // (H/G)."""
    T, H, P = x.shape
    G = B.shape[1]
    y = np.zeros((T, H, P))
    for r in range(len(cu) - 1):
        t0, t1 = int(cu[r]), int(cu[r + 1])
        for hh in range(H):
            g = hh // (H // G)
            for t in range(t0, t1):
                acc = np.zeros(P)
                if h0 is not None:
                    tot = sum(delta[q, hh] for q in range(t0, t + 1)) * A[hh]
                    acc += math.exp(tot) * (h0[r][hh] @ C[t, g])
                for s in range(t0, t + 1):
                    seg = sum(delta[q, hh] for q in range(s + 1, t + 1)) * A[hh]
                    acc += math.exp(seg) * delta[s, hh] * float(C[t, g] @ B[s, g]) * x[s, hh]
                y[t, hh] = acc + D[hh] * x[t, hh]
    return y


# ----------------------------------------------------------------------------------------
# recurrence
# ----------------------------------------------------------------------------------------
def test_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    T = len(g["x"])
    out = scan_prefill(np.array(g["x"]).reshape(T, 1, 1), np.array(g["dt"]).reshape(T, 1),
                       np.array(g["A"]), np.array(g["B"]).reshape(T, 1, 1),
                       np.array(g["C"]).reshape(T, 1, 1), np.array(g["D"]),
                       [0, T], chunk_size=64)
    np.testing.assert_allclose(out["y"].ravel(), g["y"], rtol=1e-15, atol=0)
    np.testing.assert_allclose(out["final_states"].ravel(), [g["y"][-1]], rtol=1e-15)


@pytest.mark.parametrize("seed,T,H,P,G,N,S,init", [
    (0, 9, 1, 1, 1, 1, 1, False),
    (1, 17, 2, 3, 1, 4, 1, True),
    (2, 24, 4, 2, 2, 3, 3, True),       # G = 2: heads {0,1} read group 0, {2,3} group 1
    (3, 20, 2, 4, 2, 2, 2, False),
])
def test_bruteforce_quadratic_form(seed, T, H, P, G, N, S, init):
    x, dt, A, B, C, D, cu, h0 = _rand_case(seed, T, H, P, G, N, S, init)
    out = scan_prefill(x, dt, A, B, C, D, cu, chunk_size=5, initial_states=h0)
    ref = _bruteforce_y(x, dt, A, B, C, D, cu, h0)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_A_zero_is_a_prefix_sum():
    x, dt, A, B, C, D, cu, h0 = _rand_case(5, 40, 3, 4, 1, 6, 1, True)
    A = np.zeros_like(A)
    out = scan_prefill(x, dt, A, B, C, D, cu, chunk_size=8, initial_states=h0)
    inj = (dt[:, :, None] * x)[:, :, :, None] * B[:, 0][:, None, None, :]   # [T,H,P,N]
    h = h0[0][None] + np.cumsum(inj, axis=0)
    y = np.einsum("thpn,tn->thp", h, C[:, 0]) + D[None, :, None] * x
    np.testing.assert_allclose(out["y"], y, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["final_states"][0], h[-1], rtol=1e-12, atol=1e-12)


def test_dt_zero_keeps_the_initial_state():
    x, dt, A, B, C, D, cu, h0 = _rand_case(6, 30, 2, 3, 1, 5, 2, True)
    dt = np.zeros_like(dt)
    out = scan_prefill(x, dt, A, B, C, D, cu, chunk_size=7, initial_states=h0)
    for r in range(2):
        t0, t1 = cu[r], cu[r + 1]
        np.testing.assert_array_equal(out["final_states"][r], h0[r])
        y = np.einsum("hpn,tn->thp", h0[r], C[t0:t1, 0]) + D[None, :, None] * x[t0:t1]
        np.testing.assert_allclose(out["y"][t0:t1], y, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("split", [1, 7, 16, 23])
def test_chunk_split_invariance(split):
    """Running [0, split) and then resuming [split, L) from the carried state with
    num_computed = split gives bit-identical outputs and checkpoints."""
    x, dt, A, B, C, D, cu, h0 = _rand_case(7, 40, 2, 3, 1, 4, 1, True)
    cs = 8
    full = scan_prefill(x, dt, A, B, C, D, [0, 40], cs, initial_states=h0)
    a = scan_prefill(x[:split], dt[:split], A, B[:split], C[:split], D, [0, split], cs,
                     initial_states=h0)
    b = scan_prefill(x[split:], dt[split:], A, B[split:], C[split:], D, [0, 40 - split], cs,
                     num_computed=[split], initial_states=[a["final_states"][0]])
    np.testing.assert_array_equal(np.concatenate([a["y"], b["y"]]), full["y"])
    np.testing.assert_array_equal(b["final_states"], full["final_states"])
    # every full-run checkpoint at an aligned position reappears in the split runs
    split_ends = list(a["boundary_ends"]) + [e + split for e in b["boundary_ends"]]
    split_states = np.concatenate([a["boundary_states"], b["boundary_states"]])
    for e, st in zip(full["boundary_ends"], full["boundary_states"]):
        assert e in split_ends
        np.testing.assert_array_equal(split_states[split_ends.index(e)], st)


def test_time_invariant_geometric_and_lfilter():
    """Constant delta, A, B, C, x (the time-invariant S4 case): the state is a geometric
    series, and each scalar chain is the IIR filter y = lfilter([1], [1, -a], u)."""
    T, H, P, N = 50, 2, 2, 3
    rng = np.random.default_rng(8)
    d, A = 0.3, np.array([-0.7, -2.0])
    xv, Bv, Cv = rng.standard_normal((H, P)), rng.standard_normal(N), rng.standard_normal(N)
    h0 = rng.standard_normal((H, P, N))
    x = np.broadcast_to(xv, (T, H, P)).copy()
    B = np.broadcast_to(Bv, (T, 1, N)).copy()
    C = np.broadcast_to(Cv, (T, 1, N)).copy()
    out = scan_prefill(x, np.full((T, H), d), A, B, C, np.zeros(H), [0, T], 16,
                       initial_states=[h0])
    for hh in range(H):
        a = math.exp(d * A[hh])
        k = np.arange(1, T + 1)[:, None, None]
        h = a ** k * h0[hh] + (d * np.outer(xv[hh], Bv))[None] * (1 - a ** k) / (1 - a)
        np.testing.assert_allclose(out["y"][:, hh], h @ Cv, rtol=1e-11, atol=1e-12)
        u = np.full(T, d * xv[hh, 0] * Bv[0])
        chain = scipy.signal.lfilter([1.0], [1.0, -a], u)
        # zero-initial-state chain of element (p=0, n=0): subtract the h0 contribution
        got = np.array([st[hh, 0, 0] for st in out["boundary_states"]])
        assert len(got) == T // 16 + (T % 16 > 0)
        ends = out["boundary_ends"]
        np.testing.assert_allclose(got - a ** ends * h0[hh, 0, 0], chain[ends - 1],
                                   rtol=1e-12, atol=1e-13)


def test_checkpoint_positions_are_the_chunk_cuts():
    cs = 6
    lengths, nc = [13, 4, 9], [0, 5, 11]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    x, dt, A, B, C, D, _, h0 = _rand_case(9, int(cu[-1]), 1, 2, 1, 2, 1, False)
    out = scan_prefill(x, dt, A, B, C, D, cu, cs, num_computed=nc)
    cuts, _, _ = chunk_metadata(cu, nc, cs)
    np.testing.assert_array_equal(out["boundary_ends"], cuts[1:])


# ----------------------------------------------------------------------------------------
# dt preprocessing
# ----------------------------------------------------------------------------------------
def test_softplus_of_zero_is_ln2_and_reproduces_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    raw = np.array([0.0, 0.0, -np.inf]).reshape(3, 1)     # softplus: ln2, ln2, 0
    out = scan_prefill(np.array(g["x"]).reshape(3, 1, 1), raw, np.array(g["A"]),
                       np.ones((3, 1, 1)), np.ones((3, 1, 1)), np.zeros(1), [0, 3], 64,
                       dt_softplus=True)
    np.testing.assert_allclose(out["y"].ravel(), g["y"], rtol=1e-15)


def test_dt_bias_then_softplus_then_clamp():
    dt = np.array([[-1.0, 0.0, 5.0]])
    bias = np.array([1.0, 0.0, -5.0])
    np.testing.assert_allclose(transform_dt(dt, bias, True), [[math.log(2)] * 3], rtol=1e-15)
    np.testing.assert_allclose(transform_dt(dt, None, False, 0.0, 1.0), [[0.0, 0.0, 1.0]])
    np.testing.assert_allclose(transform_dt(np.array([[800.0]]), None, True), [[800.0]])


# ----------------------------------------------------------------------------------------
# Mamba1 diagonal variant
# ----------------------------------------------------------------------------------------
def test_diag_bruteforce_and_lfilter():
    T, Hc, N = 15, 3, 4
    rng = np.random.default_rng(10)
    x = rng.standard_normal((T, Hc, 1))
    dt = np.logaddexp(0.0, rng.standard_normal((T, Hc)) - 1.0)
    A = -np.exp(rng.uniform(0, np.log(8), size=(Hc, N)))
    B = rng.standard_normal((T, 1, N))
    C = rng.standard_normal((T, 1, N))
    D = rng.standard_normal(Hc)
    out = scan_prefill(x, dt, A, B, C, D, [0, T], 4)
    for c in range(Hc):
        ref = np.zeros(T)
        for t in range(T):
            acc = 0.0
            for n in range(N):
                for s in range(t + 1):
                    seg = sum(dt[q, c] for q in range(s + 1, t + 1)) * A[c, n]
                    acc += math.exp(seg) * dt[s, c] * x[s, c, 0] * B[s, 0, n] * C[t, 0, n]
            ref[t] = acc + D[c] * x[t, c, 0]
        np.testing.assert_allclose(out["y"][:, c, 0], ref, rtol=1e-12, atol=1e-12)
    # one (channel, state) chain with constant delta is an IIR filter
    dt_c = np.full((T, Hc), 0.25)
    out2 = scan_prefill(x, dt_c, A, B, C, D, [0, T], 4)
    a = math.exp(0.25 * A[1, 2])
    chain = scipy.signal.lfilter([1.0], [1.0, -a], 0.25 * x[:, 1, 0] * B[:, 0, 2])
    np.testing.assert_allclose(out2["final_states"][0, 1, 0, 2], chain[-1], rtol=1e-12)


# ----------------------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------------------
def _decode_case(seed, B_pad=6, n_live=4, ntok=3, H=2, P=3, G=1, N=4, slots=20, null=0):
    rng = np.random.default_rng(seed)
    idx = np.full((B_pad, ntok), null, dtype=np.int64)
    idx[:n_live] = (rng.permutation(slots - 1)[:n_live * ntok] + 1).reshape(n_live, ntok)
    acc = np.ones(B_pad, dtype=np.int64)
    acc[:n_live] = rng.integers(1, ntok + 1, size=n_live)
    pool = rng.standard_normal((slots, H, P, N))
    x = rng.standard_normal((B_pad, ntok, H, P))
    dt = np.logaddexp(0, rng.standard_normal((B_pad, ntok, H)) - 1)
    A = -np.exp(rng.uniform(0, 2, size=H))
    Bm = rng.standard_normal((B_pad, ntok, G, N))
    Cm = rng.standard_normal((B_pad, ntok, G, N))
    D = rng.standard_normal(H)
    return pool, idx, acc, x, dt, A, Bm, Cm, D


def test_decode_is_prefill_continued_from_the_accepted_checkpoint():
    pool, idx, acc, x, dt, A, Bm, Cm, D = _decode_case(11)
    pool_before = pool.copy()
    y, writes = scan_decode(pool, idx, acc, x, dt, A, Bm, Cm, D, null_block_id=0)
    np.testing.assert_array_equal(pool, pool_before)           # the oracle never mutates
    assert set(y) == {0, 1, 2, 3}
    for r in range(4):
        src = pool[idx[r, acc[r] - 1]]
        ref = scan_prefill(x[r], dt[r], A, Bm[r], Cm[r], D, [0, x.shape[1]], 1,
                           initial_states=[src])
        np.testing.assert_allclose(y[r], ref["y"], rtol=1e-14, atol=1e-14)
        for j in range(x.shape[1]):
            # slot j holds the state after j+1 of this step's tokens (chunk size 1 records
            # every token)
            np.testing.assert_allclose(writes[int(idx[r, j])], ref["boundary_states"][j],
                                       rtol=1e-14, atol=1e-14)


def test_mamba1_decode_is_the_diagonal_prefill_continued():
    """Diagonal A [H, N] with P == 1 (the Mamba1 decode): each live row's step equals the
    diagonal-A prefill (pinned above by brute force and lfilter) resumed from the accepted
    checkpoint, token by token."""
    pool, idx, acc, x, dt, _, Bm, Cm, D = _decode_case(14, H=3, P=1, N=5)
    A = -np.exp(np.random.default_rng(15).uniform(-1, 2, size=(3, 5)))
    y, writes = scan_decode(pool, idx, acc, x, dt, A, Bm, Cm, D, null_block_id=0)
    assert set(y) == {0, 1, 2, 3}
    for r in range(4):
        ref = scan_prefill(x[r], dt[r], A, Bm[r], Cm[r], D, [0, x.shape[1]], 1,
                           initial_states=[pool[idx[r, acc[r] - 1]]])
        np.testing.assert_allclose(y[r], ref["y"], rtol=1e-14, atol=1e-14)
        for j in range(x.shape[1]):
            np.testing.assert_allclose(writes[int(idx[r, j])], ref["boundary_states"][j],
                                       rtol=1e-14, atol=1e-14)
    # and one state element by hand: h = exp(delta A[c, n]) h + delta x B[n]
    r, c, n = 0, 2, 3
    h = pool[idx[r, acc[r] - 1]][c, 0, n]
    for j in range(x.shape[1]):
        h = math.exp(dt[r, j, c] * A[c, n]) * h + dt[r, j, c] * x[r, j, c, 0] * Bm[r, j, 0, n]
        assert abs(writes[int(idx[r, j])][c, 0, n] - h) <= 1e-12 * max(1.0, abs(h))


def test_decode_reads_the_source_before_writing_it():
    """num_accepted = ntok makes the source the last column, which is also written: the
    step must start from the old contents."""
    pool, idx, acc, x, dt, A, Bm, Cm, D = _decode_case(12, B_pad=1, n_live=1, ntok=2)
    acc[:] = 2
    y, writes = scan_decode(pool, idx, acc, x, dt, A, Bm, Cm, D, null_block_id=0)
    ref = scan_prefill(x[0], dt[0], A, Bm[0], Cm[0], D, [0, 2], 1,
                       initial_states=[pool[idx[0, 1]]])
    np.testing.assert_allclose(y[0], ref["y"], rtol=1e-14)
    np.testing.assert_allclose(writes[int(idx[0, 1])], ref["final_states"][0], rtol=1e-14)


def test_decode_null_rows_touch_nothing():
    pool, idx, acc, x, dt, A, Bm, Cm, D = _decode_case(13, null=-1)
    idx[4:] = -1
    y, writes = scan_decode(pool, idx, acc, x, dt, A, Bm, Cm, D, null_block_id=-1)
    assert set(y) == {0, 1, 2, 3}
    assert set(writes) == set(int(v) for v in idx[:4].ravel())


# ----------------------------------------------------------------------------------------
# "all" cache mode (one state entry per cache block)

def _block_of_by_counting(t, bs):
    """Block of absolute position t, found by counting the block ends before it (no
    division)."""
    return sum(1 for e in range(1, t + 1) if e % bs == 0)


@pytest.mark.parametrize("bs", [1, 3, 4, 8])
def test_block_indices_by_walking_tokens(bs):
    nc = [0, 1, 3, 4, 5, 7, 8, 16]
    L = [1, 3, 1, 4, 11, 1, 8, 2]
    first, last_comp, last_sched = block_indices(nc, L, bs)
    for r in range(len(nc)):
        new_blocks = [_block_of_by_counting(t, bs) for t in range(nc[r], nc[r] + L[r])]
        old_blocks = [_block_of_by_counting(t, bs) for t in range(nc[r])]
        assert first[r] == min(new_blocks) and last_sched[r] == max(new_blocks)
        assert last_comp[r] == (max(old_blocks) if old_blocks else -1)


def test_block_states_are_the_states_at_block_ends():
    """Each recorded block entry is the final state of the same sequence cut right after
    that block's last token, and exactly the blocks closed by new tokens are recorded."""
    bs = 4
    x, dt, A, B, C, D, cu, h0 = _rand_case(31, 29, 2, 3, 1, 4, S=3, init=True)
    nc = [0, 6, 9]
    res = scan_prefill(x, dt, A, B, C, D, cu, 2, num_computed=nc, initial_states=h0,
                       block_size=bs)
    seen = set()
    for r, col, h in res["block_states"]:
        seen.add((r, col))
        L_cut = (col + 1) * bs - nc[r]               # new tokens up to the block's end
        t0 = cu[r]
        assert 1 <= L_cut <= cu[r + 1] - t0
        sl = slice(t0, t0 + L_cut)
        ref = scan_prefill(x[sl], dt[sl], A, B[sl], C[sl], D, [0, L_cut], 1000,
                           initial_states=[h0[r]])
        np.testing.assert_array_equal(h, ref["final_states"][0])
    expect = {(r, b) for r in range(3) for b in range(nc[r] // bs, 100)
              if nc[r] < (b + 1) * bs <= nc[r] + cu[r + 1] - cu[r]}
    assert seen == expect


def test_prefix_cache_resume_from_a_block_entry():
    """One-shot prefill vs a prefill resumed from a cached entry: resuming after a full
    block (entry last_computed = that block) and after a partial block (entry written as the
    final state of the first part, at last_scheduled) both reproduce the one-shot y and
    final state."""
    bs, T = 4, 15
    x, dt, A, B, C, D, _, _ = _rand_case(32, T, 2, 3, 2, 4)
    full = scan_prefill(x, dt, A, B, C, D, [0, T], 2, block_size=bs)
    entries = {col: h for _, col, h in full["block_states"]}
    for cut in (4, 8, 6, 9):
        first = scan_prefill(x[:cut], dt[:cut], A, B[:cut], C[:cut], D, [0, cut], 2,
                             block_size=bs)
        _, _, last_sched = block_indices([0], [cut], bs)
        cache = {col: h for _, col, h in first["block_states"]}
        cache[int(last_sched[0])] = first["final_states"][0]
        _, last_comp, _ = block_indices([cut], [T - cut], bs)
        h_in = cache[int(last_comp[0])]
        rest = scan_prefill(x[cut:], dt[cut:], A, B[cut:], C[cut:], D, [0, T - cut], 2,
                            num_computed=[cut], initial_states=[h_in], block_size=bs)
        np.testing.assert_allclose(rest["y"], full["y"][cut:], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(rest["final_states"], full["final_states"], rtol=1e-12,
                                   atol=1e-12)
        for _, col, h in rest["block_states"]:
            np.testing.assert_allclose(h, entries[col], rtol=1e-12, atol=1e-12)


def test_all_mode_decode_reads_last_computed_and_writes_last_scheduled():
    pool, _, _, x, dt, A, Bm, Cm, D = _decode_case(33, B_pad=5, ntok=1)
    rng = np.random.default_rng(34)
    idx = rng.permutation(np.arange(1, 20))[:5 * 3].reshape(5, 3)
    lc = np.array([0, 1, 2, 1, 0])
    ls = np.array([1, 1, 2, 2, 0])
    idx[4, 0] = 0                                   # padding row: its destination is null
    y, writes = scan_decode(pool, idx, None, x, dt, A, Bm, Cm, D, null_block_id=0,
                            block_idx_last_computed=lc, block_idx_last_scheduled=ls)
    assert set(y) == {0, 1, 2, 3}
    assert set(writes) == {int(idx[r, ls[r]]) for r in range(4)}
    for r in range(4):
        ref = scan_prefill(x[r], dt[r], A, Bm[r], Cm[r], D, [0, 1], 1,
                           initial_states=[pool[idx[r, lc[r]]]])
        np.testing.assert_allclose(y[r], ref["y"], rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(writes[int(idx[r, ls[r]])], ref["final_states"][0],
                                   rtol=1e-14, atol=1e-14)


# ----------------------------------------------------------------------------------------
# chunk metadata
# ----------------------------------------------------------------------------------------
def _meta_fixture(name):
    return json.load(open(os.path.join(GOLDEN, "metadata_examples.json")))[name]


@pytest.mark.parametrize("name", ["warmup_single_chunk", "partial_first_chunks"])
def test_metadata_examples(name):
    f = _meta_fixture(name)
    cu, sidx, last = chunk_metadata(f["cu_seqlens"], f["num_computed"], f["chunk_size"])
    assert cu.tolist() == f["cu_chunk_seqlens"]
    assert sidx.tolist() == f["seq_idx"]
    assert last.tolist() == f["last_chunk_indices"]


def test_metadata_first_chunk_follows_the_partial_chunk_formula():
    """The first chunk of a resumed sequence has min(cdiv(nc, cs) * cs - nc, new) tokens
    when nc is unaligned, else min(cs, new)."""
    rng = np.random.default_rng(14)
    for _ in range(300):
        cs = int(rng.choice([1, 2, 3, 4, 8, 64, 256]))
        S = int(rng.integers(1, 6))
        new = rng.integers(1, 3 * cs + 3, size=S)
        nc = rng.integers(0, 4 * cs + 2, size=S)
        cu_seq = np.concatenate([[0], np.cumsum(new)])
        cu, sidx, last = chunk_metadata(cu_seq, nc, cs)
        for r in range(S):
            first = int(np.flatnonzero(sidx == r)[0])
            length = cu[first + 1] - cu[first]
            if nc[r] % cs:
                expect = min(-(-nc[r] // cs) * cs - nc[r], new[r])
            else:
                expect = min(cs, new[r])
            assert length == expect
            # invariants: one sequence per chunk, 1 <= len <= cs, last index correct
            ks = np.flatnonzero(sidx == r)
            assert last[r] == ks[-1]
            assert cu[ks[0]] == cu_seq[r] and cu[ks[-1] + 1] == cu_seq[r + 1]
            lens = cu[ks + 1] - cu[ks]
            assert lens.min() >= 1 and lens.max() <= cs
            # every chunk but the last ends at an absolute multiple of cs
            ends_abs = cu[ks + 1] - cu_seq[r] + nc[r]
            assert np.all(ends_abs[:-1] % cs == 0)
