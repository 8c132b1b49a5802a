"""Helpers for the GPU parity tests: move seeded inputs to the device, run the HIP path
through the C ABI, and run the oracle on the same (dtype-rounded) arrays."""
from __future__ import annotations

import math

import numpy as np

from oracle import scan_decode, scan_prefill
from selective_state_space_mamba2_amd import api
from selective_state_space_mamba2_amd.inputs import bf16_from_bits

DEV = "cuda"

# Tolerances: max |got - ref| <= TOL * max |ref| per output tensor.  "f16" is for states
# stored in an fp16 pool from fp32 arithmetic: one round to nearest even (relative error at
# most 2**-11) on top of the fp32 error; a bf16 rounding (2**-9) would not pass it.
TOL = {"bf16": 2e-2, "f32": 1e-4, "f16": 1e-3}
_POOL_TORCH = {"bf16": "bfloat16", "f16": "float16"}


def torch():
    import torch as _t
    return _t


def dev_token(inp, name):
    t = torch()
    a = getattr(inp, name)
    if inp.in_dtype == "bf16":
        return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(t.bfloat16).to(DEV)
    return t.from_numpy(np.asarray(a, dtype=np.float32)).to(DEV)


def dev_f32(a):
    return torch().from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dev_i32(a):
    return torch().from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def host64(t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_close(got, ref, tol, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    assert err <= tol * scale, f"{what}: max err {err:.3e} > {tol} * {scale:.3e}"
    return err / max(scale, 1e-300)


def prefill_metadata(inp):
    return api.ssd_build_chunk_metadata(inp.cu_seqlens, inp.num_computed, inp.chunk_size)


def rounded_pool(inp, dtype):
    """Switch ``inp`` to a 2-byte state pool (``dtype`` "bf16" or "f16"): the pool values
    become their rounding to that type (round to nearest even, kept as float32 in
    ``inp.pool`` for the oracle).  Returns ``inp``."""
    t = torch()
    inp.pool = t.from_numpy(inp.pool).to(getattr(t, _POOL_TORCH[dtype])).float().numpy()
    inp.pool_dtype = dtype
    return inp


def bf16_pool(inp):
    return rounded_pool(inp, "bf16")


def f16_pool(inp):
    return rounded_pool(inp, "f16")


def pool_tol(inp):
    """Tolerance of the states written to ``inp``'s pool: the input dtype's, or the pool
    type's rounding where that is the larger."""
    return max(TOL[inp.in_dtype], TOL.get(getattr(inp, "pool_dtype", "f32"), 0.0))


def _dev_pool(inp):
    t = torch()
    pool = t.from_numpy(inp.pool).to(DEV)
    kind = getattr(inp, "pool_dtype", "f32")
    return pool if kind == "f32" else pool.to(getattr(t, _POOL_TORCH[kind]))


def run_prefill(inp, *, write_final=True, want_states=True, dt_bias=None, softplus=False,
                dt_limit=(0.0, math.inf), debug=False, use_D=True, views=False,
                y_fill=float("nan")):
    """Run ssd_prefill on ``inp``.  Returns host arrays (float64 unless noted)."""
    t = torch()
    cuc, sidx, last = prefill_metadata(inp)
    T, H, P, G, N = inp.T, inp.H, inp.P, inp.G, inp.N
    Cn = len(sidx)
    if views:
        # x, B and C as views into one projection buffer [T, H*P + 2*G*N + pad], as when
        # they come out of one split projection; y lands in a wider buffer too.
        xb, bb, cb = dev_token(inp, "x"), dev_token(inp, "B"), dev_token(inp, "C")
        width = H * P + 2 * G * N + 16
        proj = t.zeros(T, width, dtype=xb.dtype, device=DEV)
        proj[:, :H * P] = xb.reshape(T, -1)
        proj[:, H * P:H * P + G * N] = bb.reshape(T, -1)
        proj[:, H * P + G * N:H * P + 2 * G * N] = cb.reshape(T, -1)
        x = proj[:, :H * P].unflatten(1, (H, P))
        B = proj[:, H * P:H * P + G * N].unflatten(1, (G, N))
        C = proj[:, H * P + G * N:H * P + 2 * G * N].unflatten(1, (G, N))
        ybuf = t.full((T, H * P + 8), y_fill, dtype=xb.dtype, device=DEV)
        y = ybuf[:, :H * P].unflatten(1, (H, P))
        dtb = t.zeros(T, H + 8, dtype=xb.dtype, device=DEV)
        dtb[:, :H] = dev_token(inp, "dt")
        dt = dtb[:, :H]
    else:
        x, B, C, dt = (dev_token(inp, n) for n in ("x", "B", "C", "dt"))
        y = t.full_like(x, y_fill)
    A = dev_f32(inp.A)
    D = dev_f32(inp.D) if use_D else None
    pool = _dev_pool(inp) if inp.pool is not None else None
    states = t.full((Cn, H, P, N), float("nan"), device=DEV) if want_states else None
    flag = t.zeros(1, dtype=t.int32, device=DEV)
    extra = {}
    if debug:
        extra = dict(dA_cumsum_out=t.full((H, T), float("nan"), device=DEV),
                     cb_out=t.full((Cn, G, inp.chunk_size, inp.chunk_size), float("nan"),
                                   device=DEV),
                     chunk_local_states_out=t.full((Cn, H, P, N), float("nan"), device=DEV))
    api.ssd_prefill(
        x, dt, A, B, C, inp.chunk_size, dev_i32(inp.cu_seqlens), dev_i32(cuc), dev_i32(sidx),
        dev_i32(last), y=y, D=D, dt_bias=None if dt_bias is None else dev_f32(dt_bias),
        dt_softplus=softplus, dt_limit=dt_limit, state_pool=pool,
        state_indices=None if inp.state_indices is None else dev_i32(inp.state_indices),
        has_initial_state=(None if inp.has_initial_state is None
                           else dev_i32(inp.has_initial_state)),
        write_final_to_pool=write_final and pool is not None, chunk_states_out=states,
        device_error_flag=flag, **extra)
    t.cuda.synchronize()
    out = dict(y=host64(y), flag=int(flag.item()), metadata=(cuc, sidx, last))
    if states is not None:
        out["states"] = states.cpu().numpy().astype(np.float64)
    if pool is not None:
        out["pool"] = pool.float().cpu().numpy()
    for k, v in extra.items():
        out[k] = v.cpu().numpy().astype(np.float64)
    return out


def _vals(inp, name, rows, heads=None):
    """fp64 values of a token tensor restricted to token rows (and heads) before conversion."""
    a = getattr(inp, name)[rows]
    if heads is not None:
        a = a[:, heads]
    if inp.in_dtype == "bf16":
        return bf16_from_bits(a)
    return np.asarray(a, dtype=np.float64)


def oracle_prefill(inp, *, seqs=None, heads=None, dt_bias=None, softplus=False,
                   dt_limit=(0.0, math.inf), use_D=True):
    """The oracle on the same arrays, optionally restricted to some sequences (each run
    separately with its own tokens) and heads (one per group keeps the head->group map)."""
    A, D = inp.A, (inp.D if use_D else None)
    bias = dt_bias
    if heads is not None:
        heads = list(heads)
        A = A[heads]
        D = None if D is None else D[heads]
        bias = None if bias is None else np.asarray(bias)[heads]
        if inp.G > 1:
            groups = [h // (inp.H // inp.G) for h in heads]
            assert groups == list(range(len(heads))), "pick one head per group, in order"
    cu = inp.cu_seqlens
    seqs = range(inp.num_seqs) if seqs is None else seqs
    res = {}
    for r in seqs:
        t0, t1 = int(cu[r]), int(cu[r + 1])
        rows = slice(t0, t1)
        h0 = None
        if inp.has_initial_state is not None and inp.has_initial_state[r]:
            h0 = inp.pool[inp.state_indices[r]].astype(np.float64)
            if heads is not None:
                h0 = h0[heads]
        res[r] = scan_prefill(_vals(inp, "x", rows, heads), _vals(inp, "dt", rows, heads), A,
                              _vals(inp, "B", rows), _vals(inp, "C", rows), D, [0, t1 - t0],
                              inp.chunk_size, num_computed=[int(inp.num_computed[r])],
                              initial_states=[h0], dt_bias=bias, dt_softplus=softplus,
                              dt_min=dt_limit[0], dt_max=dt_limit[1])
    return res


def check_prefill(inp, got, ref, *, heads=None, tol=None, check_pool=True, pool_tol=None):
    """Compare every output of the sequences in ``ref`` (dict seq -> oracle result)."""
    tol = TOL[inp.in_dtype] if tol is None else tol
    cuc, sidx, last = got["metadata"]
    hs = slice(None) if heads is None else list(heads)
    worst = 0.0
    for r, o in ref.items():
        t0, t1 = int(inp.cu_seqlens[r]), int(inp.cu_seqlens[r + 1])
        worst = max(worst, assert_close(got["y"][t0:t1][:, hs], o["y"], tol, f"y seq {r}"))
        ks = np.flatnonzero(sidx == r)
        # the oracle's checkpoint positions are the builder's chunk ends, bit for bit
        np.testing.assert_array_equal(o["boundary_ends"] + t0, cuc[ks + 1])
        if "states" in got:
            worst = max(worst, assert_close(got["states"][ks][:, hs], o["boundary_states"], tol,
                                            f"chunk states seq {r}"))
        if check_pool and "pool" in got and inp.state_indices is not None:
            slot = int(inp.state_indices[r])
            worst = max(worst, assert_close(got["pool"][slot][hs], o["final_states"][0],
                                            tol if pool_tol is None else pool_tol,
                                            f"pool slot of seq {r}"))
    return worst


def run_decode(inp, *, y_fill=7.0, use_acc=True, dt_bias=None, softplus=False,
               dt_limit=(0.0, math.inf), num_accepted=None):
    t = torch()
    x, dt, B, C = (dev_token(inp, n) for n in ("x", "dt", "B", "C"))
    y = t.full_like(x, y_fill)
    pool = _dev_pool(inp)
    flag = t.zeros(1, dtype=t.int32, device=DEV)
    acc = inp.num_accepted if num_accepted is None else num_accepted
    api.ssd_state_update(
        x, dt, dev_f32(inp.A), B, C, pool, dev_i32(inp.state_indices), y=y,
        num_accepted_tokens=dev_i32(acc) if use_acc else None,
        null_block_id=inp.null_block_id, D=dev_f32(inp.D),
        dt_bias=None if dt_bias is None else dev_f32(dt_bias), dt_softplus=softplus,
        dt_limit=dt_limit, device_error_flag=flag)
    t.cuda.synchronize()
    return dict(y=y, pool=pool.float().cpu().numpy(), flag=int(flag.item()))


def oracle_decode(inp, rows=None, use_acc=True, dt_bias=None, softplus=False,
                  dt_limit=(0.0, math.inf), num_accepted=None):
    acc = inp.num_accepted if num_accepted is None else num_accepted
    return scan_decode(inp.pool, inp.state_indices, acc if use_acc else None,
                       inp.values("x"), inp.values("dt"), inp.A, inp.values("B"),
                       inp.values("C"), inp.D, inp.null_block_id, dt_bias=dt_bias,
                       dt_softplus=softplus, dt_min=dt_limit[0], dt_max=dt_limit[1],
                       rows=rows)
