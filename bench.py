#!/usr/bin/env python
"""Benchmark of the MI355X SSD scan path (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--primary-only]

One step is one pass of the prefill path over the Nemotron-H-like per-layer shard with
prefix caching (16 varlen sequences of 512..8192 new tokens resuming at unaligned points,
48 heads, head_dim 64, 4 groups, dstate 128, chunk 256, bf16 in / fp32 state, initial
states gathered from a 1024-slot pool, the state written at every chunk end and the final
state back to the pool): chunk metadata on the host, its copy to the device, and the two
prefill kernels.  It is the largest single-GPU SSD prefill workload, so it carries the
headline value.  Inputs are resident in HBM before timing starts; four input/output buffer
sets rotate so the 256 MB Infinity Cache cannot hold a step's working set.  The line also
carries, each with its own roofline and oracle baseline, the Mamba2-2.7B-like layer
prefill (4 x 2048 tokens, 80 heads), the tiny fp32 prefill, the decode state update (256
live requests of a 512-row padded batch, 1+3 tokens, [2048,48,64,128] fp32 pool) and the
Mamba1 long-context diagonal scan, and as further objects the prefix-cache prefill in the
all cache mode, the Mamba1 decode, the decode with a bf16 and with an fp16 state pool and the
causal conv1d prefill and decode update.

Roofline: each kernel's duration comes from HIP events the library records around its
own launches on the launch stream (the C ABI's timing hook), averaged over the timed
steps; achieved = the kernel's algorithmic bytes (or flops) per launch / that duration.
Every timed leg passes a device error flag and checks it is still zero after its timed
loop (outside the timed region).
"""
import os

# The oracle baseline runs single-threaded: set before numpy (or torch) is imported.
for _v in ("OMP_NUM_THREADS", "MKL_NUM_THREADS", "OPENBLAS_NUM_THREADS"):
    os.environ[_v] = "1"

import argparse
import gc
import hashlib
import json
import math
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA, TFLOP/s
# Vector-ALU peak: 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz = 39.3 T lane-ops/s; an FMA counts
# 2 flops (78.6 TFLOP/s); the 157.3 TFLOP/s headline needs packed FP32, which this build
# does not emit.
VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9
METRIC = "SSD prefill tokens/s (% MFMA peak) + decode state-updates/s (% HBM GB/s)"


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------------------
# algorithmic work (bytes and flops a kernel must move / do; redundant work not counted)
# ----------------------------------------------------------------------------------------
def _rw(read, write, flops=0):
    """Algorithmic bytes of a kernel, split into reads and writes."""
    return dict(bytes=read + write, read=read, write=write, flops=flops)


def prefill_work(inp, cuc, sidx, state_writes=None):
    """Algorithmic bytes (read / written) and flops per kernel.  ``state_writes``: fp32
    states written per call (default: one per chunk plus the final states; the all cache
    mode passes its block-end entries plus the final states)."""
    b = 2 if inp.in_dtype == "bf16" else 4
    T, H, P, G, N = inp.T, inp.H, inp.P, inp.G, inp.N
    S, C = inp.num_seqs, len(sidx)
    st = H * P * N * 4
    n_init = 0 if inp.has_initial_state is None else int(inp.has_initial_state.sum())
    n_final = 0 if inp.pool is None else S
    n_out = C + n_final if state_writes is None else state_writes
    lens = [int(cuc[k + 1] - cuc[k]) for k in range(C)]
    cs = inp.chunk_size
    nfrag = sum(i // 2 + 1 for i in range(cs // 16))
    frags = C * G * (nfrag * 512 + 2 * N * cs) * b
    flops_y = sum(H * (4 * l * P * N + P * l * (l + 1)) for l in lens)
    flops_cb = sum(G * N * l * (l + 1) for l in lens)
    x_b = T * H * P * b                                       # x in (and y out)
    dc = C * H * 2 * cs * 4                                   # cumsum + delta (fp32)
    # march path: the prep kernel reads dt, B and C and writes the cumsum, delta and the
    # C.B^T / B^T / C fragments; the march kernel reads x, C, the cumsum and the initial
    # states and writes y and the states (fragments come through L2)
    k_prep = _rw(T * H * b + 2 * T * G * N * b, dc + frags, flops_cb)
    k_march = _rw(x_b + T * G * N * b + dc + n_init * st, x_b + n_out * st, flops_y)
    # chain path: the prep kernel only builds the fragments; the chain kernel reads dt
    # itself (a chain also reads back its predecessor's state, through L2 or HBM: not
    # counted, it is not algorithmic)
    k_prep_chain = _rw(2 * T * G * N * b, frags, flops_cb)
    k_chain = _rw(x_b + T * G * N * b + T * H * b + n_init * st, x_b + n_out * st, flops_y)
    path = _rw(T * (H * P * b + H * b + 2 * G * N * b) + n_init * st, x_b + n_out * st,
               flops_y + flops_cb)
    return {"k_chunk_prep": k_prep, "k_chunk_march": k_march, "k_chunk_chain": k_chain,
            "k_chunk_prep/chain": k_prep_chain, "path": path}


def decode_work(inp, state_bytes=4):
    b = 2 if inp.in_dtype == "bf16" else 4
    st = inp.H * inp.P * inp.N * state_bytes
    tok_in = inp.ntok * (inp.H * inp.P * b + inp.H * b + 2 * inp.G * inp.N * b)
    tok_out = inp.ntok * inp.H * inp.P * b
    w = _rw(inp.n_live * (st + tok_in), inp.n_live * (inp.ntok * st + tok_out))
    w["updates"] = inp.n_live * inp.ntok
    return w


def diag_work(inp, C):
    b = 2 if inp.in_dtype == "bf16" else 4
    T, H, N = inp.T, inp.H, inp.N
    w = _rw(T * (2 * H * b + 2 * N * b), T * H * b + C * H * N * 4)
    w["steps"] = T * H * N
    return w


# ----------------------------------------------------------------------------------------
# device plumbing
# ----------------------------------------------------------------------------------------
def _dev_token(torch, inp, name):
    import numpy as np
    a = getattr(inp, name)
    if inp.in_dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).cuda()


class _quiet_gc:
    """Collect garbage before a timed loop and keep the collector off inside it: a
    collection of an earlier benchmark's objects during the loop stalls the host that
    issues the launches (measured: 0.6 ms per step) and would be counted as GPU time."""

    def __enter__(self):
        gc.collect()
        gc.disable()

    def __exit__(self, *exc):
        gc.enable()
        return False


def _error_flag(torch):
    """A zeroed device error word for one timed leg."""
    return torch.zeros(1, dtype=torch.int32, device="cuda")


def _assert_no_device_error(flag, what):
    """After a leg's timed loop (outside the timed region): the kernels raised no device
    error (bad metadata, an index out of range, a chain hand-off that gave up waiting)."""
    from selective_state_space_mamba2_amd.api import device_error_names
    bits = int(flag.item())
    if bits:
        raise RuntimeError(f"{what}: device error bits 0x{bits:x} "
                           f"({', '.join(device_error_names(bits))}) during the timed loop")


def _events(torch, n):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()          # materialise the underlying hipEvent_t
    return evs


def _handles(evs):
    import ctypes
    arr = (ctypes.c_void_p * len(evs))(*[e.cuda_event for e in evs])
    return arr


# Kernel-duration events are recorded on every PROFILE_EVERY-th timed step only: each
# recorded event is a marker the command processor handles between kernels, which would
# otherwise add to every step's time.
PROFILE_EVERY = 4


def _profiled(steps):
    return [i for i in range(steps) if i % PROFILE_EVERY == 0]


def _kernel_times(evs_per_step, n_kernels):
    tot = [0.0] * n_kernels
    for evs in evs_per_step:
        for i in range(n_kernels):
            tot[i] += evs[i].elapsed_time(evs[i + 1])
    return [t / len(evs_per_step) for t in tot]     # ms per launch


def _kernel_spread(evs_per_step, n_kernels):
    """p10 / median / p90 of each kernel's per-launch duration (ms) over the profiled
    steps."""
    import numpy as np
    out = []
    for i in range(n_kernels):
        d = np.array([evs[i].elapsed_time(evs[i + 1]) for evs in evs_per_step])
        out.append({"p10": round(float(np.percentile(d, 10)), 5),
                    "median": round(float(np.median(d)), 5),
                    "p90": round(float(np.percentile(d, 90)), 5)})
    return out


def _source_digest(*names):
    """Digest of kernel sources with comments and blank lines left out (a comment edit keeps
    a stored counter record valid; any code change invalidates it)."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "selective_state_space_mamba2_amd", "csrc", n)) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def _counter_traffic(kernel, workload, digest):
    """HBM bytes per launch measured with rocprofv3 PMC counters (FETCH_SIZE + WRITE_SIZE,
    each scaled by what it reads for the probe's pure-read / pure-write launches of known
    size in the same run), as recorded under profiles/.  None when no record exists or the
    kernel code changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{kernel}@{workload}")
    except (ValueError, OSError):
        return None
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec.get("bytes_per_launch")


TRAFFIC_SOURCE = ("stored record (profiles/counters.json): rocprofv3 FETCH_SIZE and WRITE_SIZE "
                  "of this kernel on this workload, each scaled by what it reads for the "
                  "library probe's pure-read / pure-write launches of known size in the same "
                  "run, keyed by a digest of the kernel code (null once it changed)")


def _roofline(bound, achieved, peak, unit, traffic=None, kernel=None, work=None):
    r = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": traffic}
    if kernel:
        r["kernel"] = kernel
    if bound == "hbm":
        r["traffic_source"] = TRAFFIC_SOURCE
        if work is not None:
            # the share of the algorithmic bytes that are reads (the measured-peak probe
            # runs at the same mix)
            r["read_frac"] = round(work["read"] / work["bytes"], 3)
    return r


# ----------------------------------------------------------------------------------------
# prefill (scalar A)
# ----------------------------------------------------------------------------------------
def all_mode_blocks(inp, cuc, sidx, last, block_size, seed=77):
    """The all cache mode's block table for a workload: distinct pool slots per (sequence,
    block), the last-computed / last-scheduled columns, and the number of block-end entries
    a call writes besides the final states."""
    import numpy as np
    S = inp.num_seqs
    nc = np.asarray(inp.num_computed, dtype=np.int64)
    L = np.diff(np.asarray(inp.cu_seqlens, dtype=np.int64))
    lc = np.where(nc > 0, (nc - 1) // block_size, -1).astype(np.int32)
    ls = ((nc + L - 1) // block_size).astype(np.int32)
    mb = int(ls.max()) + 1
    slots = inp.pool.shape[0]
    if S * mb >= slots:
        raise ValueError("pool too small for the block table")
    rng = np.random.default_rng(seed)
    table = (rng.permutation(slots - 1)[:S * mb] + 1).reshape(S, mb).astype(np.int32)
    n_blk = 0
    for k in range(len(sidx)):
        r = int(sidx[k])
        end = nc[r] + (int(cuc[k + 1]) - int(inp.cu_seqlens[r]))
        if end % block_size == 0 and k != int(last[r]):
            n_blk += 1
    return table, lc, ls, n_blk


def bench_prefill(torch, name, steps, warmup, sets=4, block_size=0, graph=False):
    """Time the prefill on a named workload.  block_size > 0 runs the all cache mode: one
    pool entry per cache block, no chunk-state output.  graph: also time the two kernels
    replayed from HIP graphs."""
    import numpy as np
    from selective_state_space_mamba2_amd import api
    from selective_state_space_mamba2_amd._abi import SSD_PREFILL_MAX_KERNELS, check, lib
    from selective_state_space_mamba2_amd.inputs import workload
    import ctypes

    inp = workload(name)
    cu_np = np.ascontiguousarray(inp.cu_seqlens, dtype=np.int32)
    nc_np = np.ascontiguousarray(inp.num_computed, dtype=np.int32)
    cuc, sidx, last = api.ssd_build_chunk_metadata(cu_np, nc_np, inp.chunk_size)
    C = len(sidx)
    S = inp.num_seqs
    A = torch.tensor(inp.A, dtype=torch.float32).cuda()
    D = torch.tensor(inp.D, dtype=torch.float32).cuda()
    pool = torch.from_numpy(inp.pool).cuda() if inp.pool is not None else None
    sidx_d = None if inp.state_indices is None else torch.from_numpy(inp.state_indices).cuda()
    hinit_d = (None if inp.has_initial_state is None
               else torch.from_numpy(inp.has_initial_state).cuda())
    base = {n: _dev_token(torch, inp, n) for n in ("x", "dt", "B", "C")}
    extra, state_writes = {}, None
    if block_size:
        table, lc, ls, n_blk = all_mode_blocks(inp, cuc, sidx, last, block_size)
        extra = dict(block_size=block_size, num_computed=torch.from_numpy(nc_np).cuda(),
                     block_idx_last_computed=torch.from_numpy(lc).cuda(),
                     block_idx_last_scheduled=torch.from_numpy(ls).cuda())
        sidx_d = torch.from_numpy(table).cuda()
        state_writes = n_blk + S
    flag = _error_flag(torch)
    bufs = []
    for i in range(sets):
        d = {n: (t if i == 0 else t.clone()) for n, t in base.items()}
        d["y"] = torch.empty_like(d["x"])
        d["states"] = (None if block_size else
                       torch.empty(C, inp.H, inp.P, inp.N, dtype=torch.float32, device="cuda"))
        # the four metadata arrays packed in one device buffer, filled by one copy per step
        d["meta"] = torch.empty(S + 1 + C + 1 + C + S, dtype=torch.int32, device="cuda")
        d["cu_seq"] = d["meta"][:S + 1]
        d["cu_chunk"] = d["meta"][S + 1:S + C + 2]
        d["seq_idx"] = d["meta"][S + C + 2:S + 2 * C + 2]
        d["last"] = d["meta"][S + 2 * C + 2:]
        d["host"] = torch.empty(S + 1 + C + 1 + C + S, dtype=torch.int32).pin_memory()
        bufs.append(d)
    args = [api.prefill_args(d["x"], d["dt"], A, d["B"], d["C"], inp.chunk_size, d["cu_seq"],
                             d["cu_chunk"], d["seq_idx"], d["last"], d["y"], D=D,
                             state_pool=pool, state_indices=sidx_d,
                             has_initial_state=hinit_d, write_final_to_pool=pool is not None,
                             chunk_states_out=None if block_size else d["states"],
                             device_error_flag=flag, **extra)
            for d in bufs]
    ws_bytes = api.ssd_prefill_workspace_size(args[0])
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    nk = ctypes.c_int32(0)
    names = (ctypes.c_char_p * SSD_PREFILL_MAX_KERNELS)()
    check("ssd_prefill_kernel_count", lib().ssd_prefill_kernel_count(ctypes.byref(args[0]),
                                                                     ctypes.byref(nk), names))
    knames = [names[i].decode() for i in range(nk.value)]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step(i, evs=None):
        d, a = bufs[i % sets], args[i % sets]
        # a0: chunk metadata on the host, then an asynchronous copy to the device
        c2, s2, l2 = api.ssd_build_chunk_metadata(cu_np, nc_np, inp.chunk_size)
        h = d["host"].numpy()
        h[:S + 1], h[S + 1:S + C + 2] = cu_np, c2
        h[S + C + 2:S + 2 * C + 2], h[S + 2 * C + 2:] = s2, l2
        d["meta"].copy_(d["host"], non_blocking=True)
        a.profile_events = None if evs is None else ctypes.cast(evs, ctypes.c_void_p)
        check("ssd_prefill", lib().ssd_prefill(ctypes.byref(a), ws.data_ptr(), ws.numel(), sp))

    for i in range(warmup):
        step(i)
    ev_sets = [_events(torch, nk.value + 1) for _ in _profiled(steps)]
    handles = [_handles(e) for e in ev_sets]
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with _quiet_gc():
        start.record()
        for i in range(steps):
            step(i, handles[i // PROFILE_EVERY] if i % PROFILE_EVERY == 0 else None)
        end.record()
        torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    _assert_no_device_error(flag, f"prefill {name}")
    kt = _kernel_times(ev_sets, nk.value)
    spread = _kernel_spread(ev_sets, nk.value)
    work = prefill_work(inp, cuc, sidx, state_writes)
    if "k_chunk_chain" in knames:
        work["k_chunk_prep"] = work.pop("k_chunk_prep/chain")
    graph_ms = None
    if graph:
        # the device part of the step (both kernels, metadata already resident) captured
        # once per buffer set in a HIP graph and replayed round-robin: no launch overhead
        graphs = []
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        for i in range(sets):
            args[i].profile_events = None
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(cap):
                with torch.cuda.graph(g, stream=cap):
                    check("ssd_prefill", lib().ssd_prefill(ctypes.byref(args[i]), ws.data_ptr(),
                                                           ws.numel(), cap.cuda_stream))
            graphs.append(g)
        stream.wait_stream(cap)
        for i in range(warmup):
            graphs[i % sets].replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with _quiet_gc():
            g0.record()
            for i in range(steps):
                graphs[i % sets].replay()
            g1.record()
            torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / steps
        _assert_no_device_error(flag, f"prefill {name} (graph replay)")
        del graphs
    return dict(inp=inp, C=C, total_ms=total_ms, ms_per_step=total_ms / steps,
                kernel_ms=dict(zip(knames, kt)), kernel_spread=dict(zip(knames, spread)),
                work=work, graph_ms=graph_ms)


def prefill_report(res, name, with_counters=True):
    inp = res["inp"]
    tok_s = inp.T / (res["ms_per_step"] * 1e-3)
    kms = res["kernel_ms"]
    dom = max(kms, key=kms.get)
    w = res["work"]
    gbs = w[dom]["bytes"] / (kms[dom] * 1e-3) / 1e9
    digest = _source_digest("ssd_prefill.hip", "ssd_device.h")
    traffic = _counter_traffic(dom, name, digest) if with_counters else None
    dev_ms = sum(kms.values())
    path_tflops = w["path"]["flops"] / (dev_ms * 1e-3) / 1e12
    path_gbs = w["path"]["bytes"] / (dev_ms * 1e-3) / 1e9
    return dict(
        tokens_per_s=tok_s,
        roofline=_roofline("hbm", gbs, HBM_PEAK_GBS, "GB/s", traffic, dom, w[dom]),
        kernels={k: {"ms": round(v, 5), "ms_spread": res["kernel_spread"][k],
                     "gb_s": round(w[k]["bytes"] / (v * 1e-3) / 1e9, 1),
                     "tflop_s": round(w[k]["flops"] / (v * 1e-3) / 1e12, 2),
                     "alg_bytes": w[k]["bytes"], "alg_flops": w[k]["flops"]}
                 for k, v in kms.items()},
        path={"device_ms": round(dev_ms, 5), "alg_bytes": w["path"]["bytes"],
              "alg_flops": w["path"]["flops"], "hbm_frac": round(path_gbs / HBM_PEAK_GBS, 4),
              "mfma_frac": round(path_tflops / MFMA_BF16_PEAK_TFLOPS, 4)},
    )


def _cpu_info():
    return {"host_logical_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "threads_env": "OMP_NUM_THREADS=MKL_NUM_THREADS=OPENBLAS_NUM_THREADS=1"}


def cpu_baseline_prefill(inp, budget_s=None, min_s=0.5):
    """The fp64 oracle timed on the GPU machine's host, on whole sequences of the workload in
    order (each with its initial state and resume point, every chunk-end state recorded)
    until ``budget_s`` of wall time is spent (None: all of them).  A batch that finishes in
    under ``min_s`` is repeated until it has run that long.  Inputs are converted from
    their storage dtype before the clock starts."""
    import numpy as np
    from oracle import scan_prefill
    from selective_state_space_mamba2_amd.inputs import bf16_from_bits
    conv = (lambda a: bf16_from_bits(a)) if inp.in_dtype == "bf16" else (lambda a: a)
    cu = [int(v) for v in inp.cu_seqlens]
    nc = [int(v) for v in inp.num_computed]
    tokens, wall, cpu, n, reps = 0, 0.0, 0.0, 0, 1
    for r in range(inp.num_seqs):
        t0, t1 = cu[r], cu[r + 1]
        x, dt, B, C = (conv(getattr(inp, k)[t0:t1]) for k in ("x", "dt", "B", "C"))
        h0 = None
        if inp.has_initial_state is not None and inp.has_initial_state[r]:
            h0 = np.asarray(inp.pool[inp.state_indices[r]], dtype=np.float64)
        w0, c0 = time.perf_counter(), time.process_time()
        scan_prefill(x, dt, inp.A, B, C, inp.D, [0, t1 - t0], inp.chunk_size,
                     num_computed=[nc[r]], initial_states=[h0])
        wall += time.perf_counter() - w0
        cpu += time.process_time() - c0
        tokens += t1 - t0
        n += 1
        if budget_s is not None and wall >= budget_s:
            break
    while wall < min_s and n == inp.num_seqs:     # a tiny batch: repeat it
        w0, c0 = time.perf_counter(), time.process_time()
        for r in range(inp.num_seqs):
            t0, t1 = cu[r], cu[r + 1]
            scan_prefill(conv(inp.x[t0:t1]), conv(inp.dt[t0:t1]), inp.A, conv(inp.B[t0:t1]),
                         conv(inp.C[t0:t1]), inp.D, [0, t1 - t0], inp.chunk_size,
                         num_computed=[nc[r]])
        wall += time.perf_counter() - w0
        cpu += time.process_time() - c0
        tokens += cu[-1]
        reps += 1
    what = "Mamba1 diagonal-A " if inp.a_kind == "diag" else ""
    return {"value": round(tokens / wall, 2), "unit": "tokens/s",
            "cores": max(1, round(cpu / wall)), "kind": "oracle",
            "sample": f"first {n} of {inp.num_seqs} sequences ({tokens // reps} tokens"
                      + (f", the batch run {reps} times" if reps > 1 else "")
                      + f"), all {inp.H} {'channels' if inp.a_kind == 'diag' else 'heads'}, "
                      f"fp64 {what}sequential recurrence with every chunk-end state; "
                      f"{wall:.1f} s wall" + ("" if budget_s is None else
                                              f" (whole sequences until {budget_s:.0f} s)"),
            **_cpu_info()}


# ----------------------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------------------
def bench_decode(torch, steps, warmup, with_cpu=True, name="decode_spec", pool="f32"):
    """One decode leg; ``pool`` is the state pool's dtype: "f32", "bf16" or "f16"."""
    import ctypes
    from selective_state_space_mamba2_amd import api
    from selective_state_space_mamba2_amd._abi import check, lib
    from selective_state_space_mamba2_amd.inputs import workload
    inp = workload(name)
    x, dt, B, C = (_dev_token(torch, inp, n) for n in ("x", "dt", "B", "C"))
    y = torch.empty_like(x)
    state_pool = torch.from_numpy(inp.pool).cuda()
    if pool != "f32":
        state_pool = state_pool.to({"bf16": torch.bfloat16, "f16": torch.float16}[pool])
    idx = torch.from_numpy(inp.state_indices).cuda()
    acc = torch.from_numpy(inp.num_accepted).cuda()
    A = torch.tensor(inp.A, dtype=torch.float32).cuda()
    D = torch.tensor(inp.D, dtype=torch.float32).cuda()
    flag = _error_flag(torch)
    a = api.decode_args(x, dt, A, B, C, y, state_pool, idx, num_accepted_tokens=acc,
                        null_block_id=inp.null_block_id, D=D, device_error_flag=flag)
    sp = torch.cuda.current_stream().cuda_stream
    for _ in range(warmup):
        check("ssd_state_update", lib().ssd_state_update(ctypes.byref(a), sp))
    ev_sets = [_events(torch, 2) for _ in _profiled(steps)]
    handles = [_handles(e) for e in ev_sets]
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with _quiet_gc():
        start.record()
        for i in range(steps):
            a.profile_events = (ctypes.cast(handles[i // PROFILE_EVERY], ctypes.c_void_p)
                                if i % PROFILE_EVERY == 0 else None)
            check("ssd_state_update", lib().ssd_state_update(ctypes.byref(a), sp))
        end.record()
        torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    _assert_no_device_error(flag, f"decode {name}")
    kms = _kernel_times(ev_sets, 1)[0]
    w = decode_work(inp, 4 if pool == "f32" else 2)
    kname = "k_state_update_diag" if inp.A.ndim == 2 else "k_state_update"
    out = {"workload": name + ("" if pool == "f32" else f" ({pool} state pool)"),
           "metric": "state-updates/s",
           "value": round(w["updates"] / (ms * 1e-3), 1), "unit": "state-updates/s",
           "ms_per_step": round(ms, 5),
           "roofline": _roofline("hbm", w["bytes"] / (kms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s",
                                 _counter_traffic(kname, name + ("" if pool == "f32" else f"/{pool}_pool"),
                                                  _source_digest("ssd_decode.hip", "ssd_device.h")),
                                 kname, w),
           "kernel_ms": round(kms, 5), "kernel_ms_spread": _kernel_spread(ev_sets, 1)[0],
           "alg_bytes": w["bytes"]}
    if with_cpu:
        from oracle import scan_decode
        from selective_state_space_mamba2_amd.inputs import bf16_from_bits
        rows = list(range(inp.n_live))     # every live row: the whole timed step
        w0, c0 = time.perf_counter(), time.process_time()
        scan_decode(inp.pool, inp.state_indices, inp.num_accepted, bf16_from_bits(inp.x),
                    bf16_from_bits(inp.dt), inp.A, bf16_from_bits(inp.B), bf16_from_bits(inp.C),
                    inp.D, inp.null_block_id, rows=rows)
        wall, cpu = time.perf_counter() - w0, time.process_time() - c0
        out["cpu_baseline"] = {"value": round(len(rows) * inp.ntok / wall, 2),
                               "unit": "state-updates/s", "cores": max(1, round(cpu / wall)),
                               "kind": "oracle",
                               "sample": f"every live row ({len(rows)}) x {inp.ntok} tokens, "
                                         f"fp64 sequential updates with the restore and every "
                                         f"checkpoint; {wall:.1f} s wall",
                               **_cpu_info()}
    del state_pool
    return out


# ----------------------------------------------------------------------------------------
# Mamba1 diagonal scan
# ----------------------------------------------------------------------------------------
def bench_diag(torch, steps, warmup, with_cpu=True, cpu_budget_s=10.0):
    import ctypes
    import numpy as np
    from selective_state_space_mamba2_amd import api
    from selective_state_space_mamba2_amd._abi import SSD_PREFILL_MAX_KERNELS, check, lib
    from selective_state_space_mamba2_amd.inputs import workload
    inp = workload("mamba1_long_diag")
    cuc, sidx, last = api.ssd_build_chunk_metadata(inp.cu_seqlens, None, inp.chunk_size)
    C = len(sidx)
    x, dt, B, Cm = (_dev_token(torch, inp, n) for n in ("x", "dt", "B", "C"))
    y = torch.empty_like(x)
    states = torch.empty(C, inp.H, 1, inp.N, dtype=torch.float32, device="cuda")
    A = torch.tensor(inp.A, dtype=torch.float32).cuda()
    D = torch.tensor(inp.D, dtype=torch.float32).cuda()
    md = [torch.from_numpy(np.asarray(v, dtype=np.int32)).cuda()
          for v in (inp.cu_seqlens, cuc, sidx, last)]
    flag = _error_flag(torch)
    a = api.prefill_args(x, dt, A, B, Cm, inp.chunk_size, *md, y, D=D, chunk_states_out=states,
                         device_error_flag=flag)
    nk = ctypes.c_int32(0)
    names = (ctypes.c_char_p * SSD_PREFILL_MAX_KERNELS)()
    check("ssd_prefill_kernel_count", lib().ssd_prefill_kernel_count(ctypes.byref(a),
                                                                     ctypes.byref(nk), names))
    kname = names[0].decode()    # the uniform or the mixed-workgroup grid
    sp = torch.cuda.current_stream().cuda_stream
    for _ in range(warmup):
        check("ssd_prefill", lib().ssd_prefill(ctypes.byref(a), None, 0, sp))
    ev_sets = [_events(torch, 2) for _ in _profiled(steps)]
    handles = [_handles(e) for e in ev_sets]
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with _quiet_gc():
        start.record()
        for i in range(steps):
            a.profile_events = (ctypes.cast(handles[i // PROFILE_EVERY], ctypes.c_void_p)
                                if i % PROFILE_EVERY == 0 else None)
            check("ssd_prefill", lib().ssd_prefill(ctypes.byref(a), None, 0, sp))
        end.record()
        torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    _assert_no_device_error(flag, "diag mamba1_long_diag")
    kms = _kernel_times(ev_sets, 1)[0]
    w = diag_work(inp, C)
    # VALU lane-ops per (token, channel, state): delta*A, exp (counted as 4: the
    # transcendental unit runs at a quarter of the FMA rate), x*B, the state FMA, the y FMA.
    lane_ops = w["steps"] * 8
    out = {"workload": "mamba1_long_diag", "metric": "tokens/s",
           "value": round(inp.T / (ms * 1e-3), 1), "unit": "tokens/s",
           "ms_per_step": round(ms, 5), "kernel_ms": round(kms, 5),
           "roofline": _roofline("alu", lane_ops / (kms * 1e-3) / 1e12,
                                 round(VALU_LANE_OPS / 1e12, 2), "T lane-op/s",
                                 _counter_traffic(kname, "mamba1_long_diag",
                                                  _source_digest("ssd_diag.hip", "ssd_device.h")),
                                 kname),
           "hbm": _roofline("hbm", w["bytes"] / (kms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s",
                            None, kname, w),
           "hbm_gb_s": round(w["bytes"] / (kms * 1e-3) / 1e9, 1), "alg_bytes": w["bytes"]}
    del x, dt, B, Cm, y
    if with_cpu:
        out["cpu_baseline"] = cpu_baseline_prefill(inp, budget_s=cpu_budget_s)
    return out


# ----------------------------------------------------------------------------------------
# causal depthwise conv1d (the step before the scan): varlen prefill and decode update
# ----------------------------------------------------------------------------------------
CONV_D = 3072        # conv channels of the pages' worked example (conv state [nb, 3, 3072])


def _conv_inputs(torch, inp):
    import numpy as np
    if inp.in_dtype == "bf16":
        x = torch.from_numpy(np.ascontiguousarray(inp.x).view(np.int16)).view(torch.bfloat16)
    else:
        x = torch.from_numpy(np.asarray(inp.x, dtype=np.float32))
    pool = torch.from_numpy(inp.pool.astype(np.float32)).cuda()
    if inp.in_dtype == "bf16":
        pool = pool.to(torch.bfloat16)
    w = torch.from_numpy(inp.weight.astype(np.float32)).cuda()
    b = torch.from_numpy(inp.bias.astype(np.float32)).cuda()
    return x.cuda(), pool, w, b


def bench_conv_prefill(torch, steps, warmup):
    """The conv over the Nemotron-H-like varlen batch (16 sequences resuming at unaligned
    points, chunk metadata of chunk 256), 3072 bf16 channels, SiLU, every conv state read
    from and written back to a 1024-slot pool."""
    import ctypes
    import numpy as np
    from selective_state_space_mamba2_amd import api
    from selective_state_space_mamba2_amd._abi import SSD_CONV_MAX_KERNELS, check, lib
    from selective_state_space_mamba2_amd.inputs import _nemotron_structure, make_conv
    lengths, nc = _nemotron_structure(2, cs=256)
    inp = make_conv(64, in_dtype="bf16", D=CONV_D, lengths=lengths, num_computed=nc,
                    pool_slots=1024, p_init=1.0)
    cuc, sidx, _ = api.ssd_build_chunk_metadata(inp.cu_seqlens, inp.num_computed, 256)
    x, pool, w, b = _conv_inputs(torch, inp)
    out = torch.empty_like(x)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    flag = _error_flag(torch)
    a = api.conv1d_args(x, w, b, out, i32(inp.cu_seqlens), i32(cuc), i32(sidx),
                        activation=True, conv_states=pool, state_indices=i32(inp.state_indices),
                        has_initial_state=i32(inp.has_initial_state), device_error_flag=flag)
    sp = torch.cuda.current_stream().cuda_stream
    for _ in range(warmup):
        check("ssd_conv1d_prefill", lib().ssd_conv1d_prefill(ctypes.byref(a), sp))
    nk = SSD_CONV_MAX_KERNELS
    ev_sets = [_events(torch, nk + 1) for _ in _profiled(steps)]
    handles = [_handles(e) for e in ev_sets]
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with _quiet_gc():
        start.record()
        for i in range(steps):
            a.profile_events = (ctypes.cast(handles[i // PROFILE_EVERY], ctypes.c_void_p)
                                if i % PROFILE_EVERY == 0 else None)
            check("ssd_conv1d_prefill", lib().ssd_conv1d_prefill(ctypes.byref(a), sp))
        end.record()
        torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    _assert_no_device_error(flag, "conv1d prefill")
    kt = _kernel_times(ev_sets, nk)
    T, D, S, W = inp.T, inp.D, len(lengths), inp.W
    # x in and out once; every sequence's old state read (all have one) and new state
    # written; the taps and bias
    st = (W - 1) * D * 2
    w_out = _rw(T * D * 2 + S * st + D * (W + 1) * 4, T * D * 2)
    k_out, k_state = w_out["bytes"], S * st
    return {"workload": f"conv1d prefill, nemotron_h_prefix_cache batch ({T} tokens, 16 "
                        f"sequences), {D} bf16 channels, width {W}, SiLU, 1024-slot pool",
            "metric": "tokens/s", "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(ms, 5),
            "roofline": _roofline("hbm", k_out / (kt[0] * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s",
                                  _counter_traffic("k_conv_prefill", "conv1d_prefill",
                                                   _source_digest("ssd_conv.hip", "ssd_device.h")),
                                  "k_conv_prefill", w_out),
            "kernels": {"k_conv_prefill": {"ms": round(kt[0], 5), "alg_bytes": k_out},
                        "k_conv_state": {"ms": round(kt[1], 5), "alg_bytes": k_state}}}


def bench_conv_update(torch, steps, warmup):
    """One decode step of the conv: 256 live rows of a 512-row padded batch, 1 input each,
    3072 bf16 channels, SiLU, a 2048-slot pool."""
    import ctypes
    import numpy as np
    from selective_state_space_mamba2_amd import api
    from selective_state_space_mamba2_amd._abi import check, lib
    from selective_state_space_mamba2_amd.inputs import make_conv
    B_pad, n_live, ntok, slots = 512, 256, 1, 2048
    inp = make_conv(68, in_dtype="bf16", D=CONV_D, lengths=[ntok] * B_pad, pool_slots=slots)
    rng = np.random.default_rng(69)
    idx = np.zeros(B_pad, dtype=np.int32)
    idx[:n_live] = rng.permutation(np.arange(1, slots))[:n_live]
    x, pool, w, b = _conv_inputs(torch, inp)
    x = x.reshape(B_pad, ntok, inp.D)
    out = torch.empty_like(x)
    flag = _error_flag(torch)
    a = api.conv1d_update_args(x, w, b, out, pool, torch.from_numpy(idx).cuda(),
                               activation=True, null_block_id=0, device_error_flag=flag)
    sp = torch.cuda.current_stream().cuda_stream
    for _ in range(warmup):
        check("ssd_conv1d_update", lib().ssd_conv1d_update(ctypes.byref(a), sp))
    ev_sets = [_events(torch, 2) for _ in _profiled(steps)]
    handles = [_handles(e) for e in ev_sets]
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with _quiet_gc():
        start.record()
        for i in range(steps):
            a.profile_events = (ctypes.cast(handles[i // PROFILE_EVERY], ctypes.c_void_p)
                                if i % PROFILE_EVERY == 0 else None)
            check("ssd_conv1d_update", lib().ssd_conv1d_update(ctypes.byref(a), sp))
        end.record()
        torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    _assert_no_device_error(flag, "conv1d update")
    kms = _kernel_times(ev_sets, 1)[0]
    D, W = inp.D, inp.W
    w_upd = _rw(n_live * ((W - 1) * D * 2 + ntok * D * 2) + D * (W + 1) * 4,
                n_live * ((W - 1) * D * 2 + ntok * D * 2))
    alg = w_upd["bytes"]
    return {"workload": f"conv1d update, {n_live} live rows of {B_pad}, {ntok} input each, "
                        f"{D} bf16 channels, SiLU, {slots}-slot pool",
            "metric": "rows/s", "value": round(n_live / (ms * 1e-3), 1), "unit": "rows/s",
            "ms_per_step": round(ms, 5), "kernel_ms": round(kms, 5),
            "roofline": _roofline("hbm", alg / (kms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s",
                                  _counter_traffic("k_conv_update", "conv1d_update",
                                                   _source_digest("ssd_conv.hip", "ssd_device.h")),
                                  "k_conv_update", w_upd),
            "alg_bytes": alg}


def _read_fracs(obj, out=None):
    """Every HBM roofline's read fraction in the line."""
    out = set() if out is None else out
    if isinstance(obj, dict):
        if obj.get("bound") == "hbm" and "read_frac" in obj:
            out.add(round(obj["read_frac"], 2))
        for v in obj.values():
            _read_fracs(v, out)
    return out


def measured_peaks(torch, read_fracs, mib=2048, reps=10, form_reps=3):
    """What this GPU sustains, as a second scale beside the spec peaks: the library's own
    streaming probe (ssd_probe_stream) moving ``mib`` MiB per launch as pure reads, pure
    writes, and at each read/write mix an HBM roofline of the line has; and a square bf16
    GEMM of 8192 through torch (hipBLASLt) for the MFMA side.  Each mix is timed in the
    probe's first access form (best of ``reps`` launches; these runs come first and in this
    order, pure reads then pure writes, which the counter calibration relies on), then in
    its eleven other forms (best of ``form_reps`` each); the rate reported is the best of
    all."""
    import ctypes
    from selective_state_space_mamba2_amd._abi import check, lib
    nbytes = mib * (1 << 20)
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").normal_()
    dst = torch.empty_like(src)
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    sp = torch.cuda.current_stream().cuda_stream

    def rate(rb, wb, form, n):
        rb, wb = rb // 16 * 16, wb // 16 * 16
        ts = []
        for i in range(n + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            check("ssd_probe_stream", lib().ssd_probe_stream(src.data_ptr(), rb, dst.data_ptr(),
                                                             wb, sink.data_ptr(), form, sp))
            e1.record()
            torch.cuda.synchronize()
            if i:
                ts.append(e0.elapsed_time(e1))
        return round((rb + wb) / (min(ts) * 1e-3) / 1e9, 1)

    mixes = [("read_gb_s", nbytes, 0), ("write_gb_s", 0, nbytes),
             ("copy_gb_s", nbytes // 2, nbytes // 2)]
    mixes += [(f"{f:.2f}", int(nbytes * f), int(nbytes * (1 - f))) for f in sorted(read_fracs)]
    best = {k: (rate(rb, wb, 0, reps), 0) for k, rb, wb in mixes}
    for form in range(1, 12):
        for k, rb, wb in mixes:
            r = rate(rb, wb, form, form_reps)
            if r > best[k][0]:
                best[k] = (r, form)
    out = {k: best[k][0] for k in ("read_gb_s", "write_gb_s", "copy_gb_s")}
    out["mix_gb_s"] = {k: best[k][0] for k, _, _ in mixes[3:]}
    out["probe_forms"] = {k: v[1] for k, v in best.items()}
    del src, dst
    m = 8192
    x = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    y = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    z = torch.empty(m, m, device="cuda", dtype=torch.bfloat16)
    torch.matmul(x, y, out=z)
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.matmul(x, y, out=z)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    out["bf16_gemm_tflop_s"] = round(2 * m ** 3 / (min(ts) * 1e-3) / 1e12, 1)
    out["note"] = (f"ssd_probe_stream (this library's streaming kernel) moving {mib} MiB per "
                   f"launch: pure reads, pure writes, a half/half copy mix and each read "
                   f"fraction (mix_gb_s keys) an HBM roofline of this line has, each the best "
                   f"of its twelve access forms (probe_forms: the winning one; contiguous or "
                   f"strided shares, non-temporal or plain stores, 2048/4096/8192 "
                   f"workgroups); torch bf16 GEMM {m}^3")
    del x, y, z
    torch.cuda.empty_cache()
    return out


def _add_measured_frac(obj, peaks):
    """Beside each HBM roofline's spec fraction, its fraction of the best rate the probe
    reached in this run over every mix it ran (pure reads, pure writes, the copy and each
    leg's own mix: a kernel's mix can run faster than the probe's interleaving of the same
    mix, so the leg's own mix alone is no ceiling); the probe's rate at the leg's own mix is
    given beside it."""
    best = max([peaks["read_gb_s"], peaks["write_gb_s"], peaks["copy_gb_s"],
                *peaks["mix_gb_s"].values()])
    if isinstance(obj, dict):
        r = obj.get("roofline")
        for cand in (obj, r):
            if isinstance(cand, dict) and cand.get("bound") == "hbm" and "read_frac" in cand:
                cand["measured_peak"] = best
                cand["measured_frac"] = round(cand["achieved"] / best, 4)
                mix = peaks["mix_gb_s"].get(f"{round(cand['read_frac'], 2):.2f}")
                if mix:
                    cand["probe_at_this_mix_gb_s"] = mix
        for v in obj.values():
            if isinstance(v, dict) and v is not r:
                _add_measured_frac(v, peaks)


def _prefill_config(inp, C):
    lens = [int(v) for v in (inp.cu_seqlens[1:] - inp.cu_seqlens[:-1])]
    nc = [int(v) for v in inp.num_computed]
    cfg = {"num_seqs": inp.num_seqs, "tokens": inp.T, "chunks": C,
           "seq_len": lens[0] if len(set(lens)) == 1 else f"{min(lens)}..{max(lens)} (varlen)",
           "nheads": inp.H, "headdim": inp.P, "ngroups": inp.G, "dstate": inp.N,
           "chunk_size": inp.chunk_size, "in_dtype": inp.in_dtype, "state_dtype": "f32",
           "states": "every chunk end" + (" + final state to the pool" if inp.pool is not None else "")}
    if any(nc):
        cfg["num_computed"] = f"{min(nc)}..{max(nc)}, none a multiple of the chunk size"
    if inp.pool is not None:
        cfg["initial_states"] = f"gathered from a {inp.pool.shape[0]}-slot fp32 pool"
    return cfg


def prefill_leg(torch, name, steps, warmup, graph=False, with_cpu=True, cpu_budget_s=None,
                block_size=0):
    """One prefill workload: timing, roofline, kernels, path totals, optional graph replay
    and the oracle baseline."""
    res = bench_prefill(torch, name, steps, warmup, graph=graph, block_size=block_size)
    key = name + ("/all" if block_size else "")
    rep = prefill_report(res, key)
    inp = res["inp"]
    out = {"workload": name + (", all cache mode (block_size 256, one pool entry per block, "
                               "no chunk-state output)" if block_size else ""),
           "metric": "tokens/s", "value": round(rep["tokens_per_s"], 1), "unit": "tokens/s",
           "ms_per_step": round(res["ms_per_step"], 5), "config": _prefill_config(inp, res["C"]),
           "roofline": rep["roofline"], "kernels": rep["kernels"], "path": rep["path"]}
    if res["graph_ms"] is not None:
        out["graph"] = {"ms_per_step": round(res["graph_ms"], 5),
                        "tokens_per_s": round(inp.T / (res["graph_ms"] * 1e-3), 1),
                        "note": "the two prefill kernels replayed from HIP graphs (metadata "
                                "resident); value is the eager step with host metadata"}
    del res
    if with_cpu:
        _log(f"cpu baseline (oracle) {name}")
        out["cpu_baseline"] = cpu_baseline_prefill(inp, budget_s=cpu_budget_s)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--primary-only", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle time per sampled baseline")
    ap.add_argument("--legs", default="",
                    help="comma-separated keys of the further workloads to run (default: all; "
                         "e.g. prefill_mamba2_2.7b,decode)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    cpu = not args.no_cpu_baseline

    name = "nemotron_h_prefix_cache"
    _log(f"prefill {name}: {args.steps} steps after {args.warmup} warm-up")
    head = prefill_leg(torch, name, args.steps, args.warmup, graph=True, with_cpu=cpu,
                       cpu_budget_s=args.cpu_budget)
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, **head["config"], "parallelism": "single GPU"},
        "roofline": head["roofline"],
        "kernels": head["kernels"],
        "path": head["path"],
        "graph": head["graph"],
    }
    if "cpu_baseline" in head:
        line["cpu_baseline"] = head["cpu_baseline"]
    if not args.primary_only:
        legs = [
            ("prefill_mamba2_2.7b", "mamba2_2.7b_prefill",
             lambda: prefill_leg(torch, "mamba2_2.7b_prefill", args.steps, args.warmup,
                                 graph=True, with_cpu=cpu)),
            ("prefill_tiny_fp32", "tiny_fp32",
             lambda: prefill_leg(torch, "tiny_fp32", args.steps, args.warmup, with_cpu=cpu)),
            ("decode", "decode_spec",
             lambda: bench_decode(torch, args.steps, args.warmup, with_cpu=cpu)),
            ("diag", "mamba1_long_diag",
             lambda: bench_diag(torch, max(3, args.steps // 5), max(1, args.warmup // 5),
                                with_cpu=cpu, cpu_budget_s=args.cpu_budget)),
            ("prefill_nemotron_all_mode", "nemotron_h_prefix_cache, all cache mode",
             lambda: prefill_leg(torch, "nemotron_h_prefix_cache", args.steps, args.warmup,
                                 with_cpu=False, block_size=256)),
            ("decode_mamba1", "mamba1_decode_spec",
             lambda: bench_decode(torch, args.steps, args.warmup, with_cpu=cpu,
                                  name="mamba1_decode_spec")),
            ("decode_bf16_pool", "decode_spec, bf16 state pool",
             lambda: bench_decode(torch, args.steps, args.warmup, with_cpu=False,
                                  pool="bf16")),
            ("decode_f16_pool", "decode_spec, fp16 state pool",
             lambda: bench_decode(torch, args.steps, args.warmup, with_cpu=False,
                                  pool="f16")),
            ("conv1d_prefill", "conv1d prefill",
             lambda: bench_conv_prefill(torch, args.steps, args.warmup)),
            ("conv1d_update", "conv1d update",
             lambda: bench_conv_update(torch, args.steps, args.warmup)),
        ]
        if args.legs:
            want = set(args.legs.split(","))
            unknown = want - {k for k, _, _ in legs}
            if unknown:
                print(f"unknown --legs entries: {sorted(unknown)}", file=sys.stderr)
                sys.exit(2)
            legs = [leg for leg in legs if leg[0] in want]
        # a secondary measurement that fails (an exception, not a device fault) is recorded
        # as such and does not cost the line the others
        for key, what, fn in legs:
            _log(what)
            try:
                line[key] = fn()
            except Exception as e:   # noqa: BLE001
                line[key] = {"workload": what, "error": f"{type(e).__name__}: {e}"}
            torch.cuda.empty_cache()
        _log("measured peaks")
        try:
            if args.legs and not _read_fracs(line):
                raise RuntimeError("no HBM roofline to compare")
            peaks = measured_peaks(torch, _read_fracs(line))
            line["measured_peaks"] = peaks
            _add_measured_frac(line, peaks)
        except Exception as e:   # noqa: BLE001
            line["measured_peaks"] = {"error": f"{type(e).__name__}: {e}"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
