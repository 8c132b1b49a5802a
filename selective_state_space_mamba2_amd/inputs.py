"""Seeded synthetic inputs for the SSD scan workloads.

This module only draws random numbers and rounds them to the storage dtype.  It holds
none of the scan's arithmetic, so the fp64 oracle and the HIP path can both consume the
exact same arrays.  Every array that is stored as bf16 is returned twice: as float64
values that are exactly representable in bf16, and (through ``bf16_bits``) as the raw
uint16 bit patterns the device receives.

Value recipe (the same for every workload unless a workload says otherwise):
  x, B, C ~ N(0, 1);  dt = softplus(N(0, 1) - 2);  A = -exp(U(log 1, log 16));  D ~ N(0, 1);
  initial / pool states ~ N(0, 0.1) (standard deviation 0.1), stored fp32.

Draw order inside one workload: sequence structure (lengths, num_computed, slot
indices, num_accepted) first, then A, D, dt, x, B, C, then the state pool.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "bf16_round", "bf16_bits", "bf16_from_bits", "PrefillInputs", "DecodeInputs",
    "make_prefill", "make_decode", "WORKLOADS", "workload",
]


# ----------------------------------------------------------------------------------------
# bf16 storage helpers (round-to-nearest-even of the fp32 bit pattern)
# ----------------------------------------------------------------------------------------
def _f32_to_bf16_bits(a32: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = np.isnan(a32)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns of ``a`` (rounded fp64 -> fp32 -> bf16, nearest-even)."""
    return _f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def bf16_from_bits(bits: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Exact values of bf16 bit patterns."""
    u = bits.astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(dtype)


def bf16_round(a: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Values of ``a`` after rounding to bf16 (returned exactly, in ``dtype``)."""
    return bf16_from_bits(bf16_bits(a), dtype)


def _store(a: np.ndarray, in_dtype: str) -> np.ndarray:
    """Round a freshly drawn array to the storage dtype and return its exact fp64 values
    (fp32 workloads) or its bf16 bit patterns (bf16 workloads)."""
    if in_dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if in_dtype == "bf16":
        return bf16_bits(a)
    raise ValueError(in_dtype)


def _softplus(z: np.ndarray) -> np.ndarray:
    # Input recipe only: dt is drawn as softplus(N(0,1) - 2), i.e. log(1 + e^z).
    return np.logaddexp(0.0, z)


# ----------------------------------------------------------------------------------------
# containers
# ----------------------------------------------------------------------------------------
@dataclasses.dataclass
class PrefillInputs:
    """One varlen prefill batch.  Token tensors are either fp64 (exact fp32 values, for
    ``in_dtype == 'f32'``) or uint16 bf16 bit patterns (``in_dtype == 'bf16'``)."""
    in_dtype: str
    T: int
    H: int
    P: int
    G: int
    N: int
    chunk_size: int
    a_kind: str                      # "scalar" (A[H]) or "diag" (A[H, N], P == 1)
    cu_seqlens: np.ndarray           # int32 [S+1]
    num_computed: np.ndarray         # int32 [S]
    A: np.ndarray                    # fp32 values (float64 array), [H] or [H, N]
    D: np.ndarray                    # fp32 values, [H]
    dt: np.ndarray                   # [T, H]
    x: np.ndarray                    # [T, H, P]
    B: np.ndarray                    # [T, G, N]
    C: np.ndarray                    # [T, G, N]
    has_initial_state: Optional[np.ndarray]   # int32 [S] or None
    state_indices: Optional[np.ndarray]       # int32 [S] or None
    pool: Optional[np.ndarray]                # float32 [slots, H, P, N] or None

    @property
    def num_seqs(self) -> int:
        return len(self.cu_seqlens) - 1

    def values(self, name: str) -> np.ndarray:
        """fp64 values of a token tensor, whatever its storage dtype."""
        a = getattr(self, name)
        if self.in_dtype == "bf16" and name in ("dt", "x", "B", "C"):
            return bf16_from_bits(a)
        return np.asarray(a, dtype=np.float64)


@dataclasses.dataclass
class DecodeInputs:
    """One padded decode batch of ``B_pad`` rows with ``ntok`` tokens per row."""
    in_dtype: str
    B_pad: int
    n_live: int
    ntok: int
    H: int
    P: int
    G: int
    N: int
    null_block_id: int
    A: np.ndarray                    # fp32 values [H], or [H, N] for a diagonal A (P == 1)
    D: np.ndarray                    # fp32 values [H]
    dt: np.ndarray                   # [B_pad, ntok, H]
    x: np.ndarray                    # [B_pad, ntok, H, P]
    B: np.ndarray                    # [B_pad, ntok, G, N]
    C: np.ndarray                    # [B_pad, ntok, G, N]
    state_indices: np.ndarray        # int32 [B_pad, ntok]
    num_accepted: np.ndarray         # int32 [B_pad]
    pool: np.ndarray                 # float32 [slots, H, P, N]

    def values(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if self.in_dtype == "bf16" and name in ("dt", "x", "B", "C"):
            return bf16_from_bits(a)
        return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------------------
# generators
# ----------------------------------------------------------------------------------------
def _draw_normal(rng: np.random.Generator, shape, big: bool) -> np.ndarray:
    # Large arrays are drawn directly in fp32 to keep host memory bounded.
    if big:
        return rng.standard_normal(shape, dtype=np.float32)
    return rng.standard_normal(shape)


def make_prefill(seed: int, *, in_dtype: str, H: int, P: int, G: int, N: int,
                 chunk_size: int, lengths, num_computed=None, a_kind: str = "scalar",
                 init: str = "none", pool_slots: int = 0, A_range=(1.0, 16.0),
                 A_zero: bool = False, dt_zero: bool = False) -> PrefillInputs:
    """Draw one prefill batch.

    ``lengths``: new tokens per sequence (list of ints).  ``num_computed``: tokens already
    processed per sequence (list, default zeros).  ``init``: "none" (zero initial states),
    or "pool" (every sequence gathers its initial state from a ``pool_slots``-slot fp32
    pool through distinct random indices in [1, pool_slots); slot 0 is never used).
    ``A_range``: A = -exp(U(log lo, log hi)).  ``A_zero`` / ``dt_zero`` force A = 0 or
    dt = 0 (degenerate cases).
    """
    rng = np.random.default_rng(seed)
    lengths = [int(v) for v in lengths]
    S = len(lengths)
    if num_computed is None:
        num_computed = [0] * S
    cu = np.zeros(S + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    has_init = state_idx = pool = None
    if init == "pool":
        if pool_slots < S + 1:
            raise ValueError("pool too small")
        state_idx = (rng.permutation(pool_slots - 1)[:S] + 1).astype(np.int32)
        has_init = np.ones(S, dtype=np.int32)
    elif init != "none":
        raise ValueError(init)

    a_shape = (H,) if a_kind == "scalar" else (H, N)
    lo, hi = A_range
    A = -np.exp(rng.uniform(np.log(lo), np.log(hi), size=a_shape))
    if A_zero:
        A = np.zeros(a_shape)
    A = A.astype(np.float32).astype(np.float64)
    D = rng.standard_normal(H).astype(np.float32).astype(np.float64)
    big = T * H * P > (1 << 24)
    dt = _softplus(_draw_normal(rng, (T, H), big).astype(np.float64) - 2.0)
    if dt_zero:
        dt = np.zeros_like(dt)
    x = _draw_normal(rng, (T, H, P), big)
    Bm = _draw_normal(rng, (T, G, N), big)
    Cm = _draw_normal(rng, (T, G, N), big)
    if init == "pool":
        pool = (rng.standard_normal((pool_slots, H, P, N), dtype=np.float32)
                * np.float32(0.1))
    return PrefillInputs(
        in_dtype=in_dtype, T=T, H=H, P=P, G=G, N=N, chunk_size=chunk_size, a_kind=a_kind,
        cu_seqlens=cu, num_computed=np.asarray(num_computed, dtype=np.int32),
        A=A, D=D, dt=_store(dt, in_dtype), x=_store(x, in_dtype), B=_store(Bm, in_dtype),
        C=_store(Cm, in_dtype), has_initial_state=has_init, state_indices=state_idx,
        pool=pool)


def make_decode(seed: int, *, in_dtype: str = "bf16", B_pad: int, n_live: int, ntok: int,
                H: int, P: int, G: int, N: int, pool_slots: int,
                null_block_id: int = 0, a_kind: str = "scalar") -> DecodeInputs:
    """Draw one padded decode batch: rows [0, n_live) are live, the tail rows are padding
    whose state_indices are all ``null_block_id``.  Live rows get distinct slot indices
    drawn from [1, pool_slots) (slot 0 is reserved), num_accepted ~ U{1..ntok}.
    ``a_kind`` "diag" draws A per (channel, state), [H, N] (the Mamba1 layout, P == 1)."""
    rng = np.random.default_rng(seed)
    if n_live * ntok > pool_slots - 1:
        raise ValueError("pool too small for distinct indices")
    idx = np.full((B_pad, ntok), null_block_id, dtype=np.int32)
    idx[:n_live] = (rng.permutation(pool_slots - 1)[:n_live * ntok] + 1).reshape(n_live, ntok)
    num_acc = np.ones(B_pad, dtype=np.int32)
    num_acc[:n_live] = rng.integers(1, ntok + 1, size=n_live)
    a_shape = (H,) if a_kind == "scalar" else (H, N)
    A = (-np.exp(rng.uniform(np.log(1.0), np.log(16.0), size=a_shape))).astype(np.float32).astype(np.float64)
    D = rng.standard_normal(H).astype(np.float32).astype(np.float64)
    dt = _softplus(rng.standard_normal((B_pad, ntok, H)) - 2.0)
    x = rng.standard_normal((B_pad, ntok, H, P))
    Bm = rng.standard_normal((B_pad, ntok, G, N))
    Cm = rng.standard_normal((B_pad, ntok, G, N))
    pool = rng.standard_normal((pool_slots, H, P, N), dtype=np.float32) * np.float32(0.1)
    return DecodeInputs(
        in_dtype=in_dtype, B_pad=B_pad, n_live=n_live, ntok=ntok, H=H, P=P, G=G, N=N,
        null_block_id=null_block_id, A=A, D=D, dt=_store(dt, in_dtype),
        x=_store(x, in_dtype), B=_store(Bm, in_dtype), C=_store(Cm, in_dtype),
        state_indices=idx, num_accepted=num_acc, pool=pool)


# ----------------------------------------------------------------------------------------
# the named workloads
# ----------------------------------------------------------------------------------------
def _nemotron_structure(seed: int, n_seqs: int = 16, cs: int = 256):
    """Varlen lengths L ~ U{512..8192} and num_computed ~ U{0..4096} redrawn until it is
    not a multiple of the chunk size (so every first chunk is partial)."""
    rng = np.random.default_rng(10_000 + seed)
    lengths = rng.integers(512, 8192 + 1, size=n_seqs)
    nc = []
    for _ in range(n_seqs):
        v = int(rng.integers(0, 4096 + 1))
        while v % cs == 0:
            v = int(rng.integers(0, 4096 + 1))
        nc.append(v)
    return [int(v) for v in lengths], nc


@dataclasses.dataclass
class ConvInputs:
    """A causal conv1d batch: x [T, D] (stored like the prefill token tensors), weight
    [D, W] and bias [D] (exact fp32 values), a conv-state pool [slots, W-1, D] of values
    rounded to the input dtype (fp64 here), one slot per sequence and has_initial_state."""
    in_dtype: str
    T: int
    D: int
    W: int
    cu_seqlens: np.ndarray
    num_computed: np.ndarray
    x: np.ndarray
    weight: np.ndarray
    bias: np.ndarray
    pool: np.ndarray
    state_indices: np.ndarray
    has_initial_state: np.ndarray

    def values(self, a: np.ndarray) -> np.ndarray:
        return bf16_from_bits(a) if self.in_dtype == "bf16" else np.asarray(a, dtype=np.float64)


def make_conv(seed: int, *, in_dtype: str, D: int, lengths, num_computed=None, W: int = 4,
              pool_slots: int = 0, p_init: float = 0.5) -> ConvInputs:
    """Draw one conv1d batch: x ~ N(0, 1), weight ~ N(0, 1/W), bias ~ N(0, 0.1), pool
    states ~ N(0, 1) rounded to the input dtype, distinct slots in [1, pool_slots),
    has_initial_state ~ Bernoulli(p_init)."""
    rng = np.random.default_rng(seed)
    lengths = [int(v) for v in lengths]
    S = len(lengths)
    cu = np.zeros(S + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    nc = np.zeros(S, dtype=np.int32) if num_computed is None else np.asarray(num_computed, dtype=np.int32)
    x = _store(_draw_normal(rng, (T, D), T * D > (1 << 24)), in_dtype)
    weight = (rng.standard_normal((D, W)) / np.sqrt(W)).astype(np.float32).astype(np.float64)
    bias = (0.1 * rng.standard_normal(D)).astype(np.float32).astype(np.float64)
    slots = max(pool_slots, S + 1)
    pool = rng.standard_normal((slots, W - 1, D), dtype=np.float32)
    pool = bf16_round(pool) if in_dtype == "bf16" else pool.astype(np.float64)
    sidx = (rng.permutation(slots - 1)[:S] + 1).astype(np.int32)
    has_init = (rng.uniform(size=S) < p_init).astype(np.int32)
    return ConvInputs(in_dtype=in_dtype, T=T, D=D, W=W, cu_seqlens=cu, num_computed=nc, x=x,
                      weight=weight, bias=bias, pool=pool, state_indices=sidx,
                      has_initial_state=has_init)


def workload(name: str, seed: Optional[int] = None):
    """Build one of the named workloads (full size).  Returns PrefillInputs or
    DecodeInputs."""
    spec = WORKLOADS[name]
    s = spec["seed"] if seed is None else seed
    if spec["kind"] == "decode":
        kw = {k: v for k, v in spec.items() if k not in ("kind", "seed")}
        return make_decode(s, **kw)
    kw = {k: v for k, v in spec.items() if k not in ("kind", "seed", "structure")}
    if spec.get("structure") == "nemotron":
        lengths, nc = _nemotron_structure(s, cs=spec["chunk_size"])
        kw["lengths"], kw["num_computed"] = lengths, nc
    return make_prefill(s, **kw)


WORKLOADS = {
    # 1 sequence, L=256, fp32, zero initial state, states at each chunk boundary.
    "tiny_fp32": dict(kind="prefill", seed=0, in_dtype="f32", H=4, P=16, G=1, N=16,
                      chunk_size=64, lengths=[256]),
    # Mamba2-2.7B-like layer: 4 packed sequences of 2048 tokens, bf16 in, fp32 state.
    "mamba2_2.7b_prefill": dict(kind="prefill", seed=1, in_dtype="bf16", H=80, P=64, G=1,
                                N=128, chunk_size=256, lengths=[2048] * 4),
    # Nemotron-H-like per-layer shard, 16 varlen sequences resuming from a 1024-slot pool.
    "nemotron_h_prefix_cache": dict(kind="prefill", seed=2, in_dtype="bf16", H=48, P=64,
                                    G=4, N=128, chunk_size=256, structure="nemotron",
                                    lengths=None, init="pool", pool_slots=1024),
    # Decode: pool [2048,48,64,128], 256 live rows of a 512-row graph batch, 1+3 tokens.
    "decode_spec": dict(kind="decode", seed=3, in_dtype="bf16", B_pad=512, n_live=256,
                        ntok=4, H=48, P=64, G=4, N=128, pool_slots=2048, null_block_id=0),
    # Mamba1-style decode: pool [1024,5120,1,16], 256 live rows of a 512-row batch, 1+3
    # tokens, diagonal A.
    "mamba1_decode_spec": dict(kind="decode", seed=5, in_dtype="bf16", B_pad=512, n_live=256,
                               ntok=4, H=5120, P=1, G=1, N=16, pool_slots=1025,
                               null_block_id=0, a_kind="diag"),
    # Mamba1-style diagonal scan: d_inner=5120, dstate=16, 8 x 16384 tokens, cs=2048.
    "mamba1_long_diag": dict(kind="prefill", seed=4, in_dtype="bf16", H=5120, P=1, G=1,
                             N=16, chunk_size=2048, lengths=[16384] * 8, a_kind="diag"),
}
