"""Plain, slow, fp64 CPU oracle for the Mamba2 SSD scan path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute this
module: only the test suite, the package smoke check and the benchmark's CPU-baseline leg
use it.  It shares no code with the HIP library (no kernels, headers, helpers, tables or
pre/post-processing); its inputs come from the seeded generators in
``selective_state_space_mamba2_amd/inputs.py``, which hold none of the scan's arithmetic.

What it computes, and where that is defined
------------------------------------------
* The selective state-space recurrence ("[vLLM] Mamba (SSM): linear-time sequence
  modeling", intro and "paper key content": an O(n) linear recurrence replaces O(n^2)
  attention, and the S6 model makes Delta, B and C functions of the input, one value per
  token).  Per head h, with a state h_t in R^{P x N} (the pool stores states as
  (num_heads, head_dim, state_size): "vLLM v0.20.0 adds disaggregated serving for hybrid
  SSM models", section on why FA and SSM state differ):

      a_t    = exp(delta_t * A_h)                                    (state decay)
      h_t    = a_t * h_{t-1} + delta_t * x_t B_t^T                   (x_t in R^P, B_t in R^N)
      y_t    = h_t C_t + D_h * x_t                                   (C_t in R^N)

  Heads map onto B/C groups in contiguous blocks, g(h) = h // (H / G) (the warm-up code
  of "vLLM Mamba2 SSD kernel warm-up", mamba_mixer2.py section, divides both nheads and
  ngroups by the tensor-parallel size).
* The Mamba1 variant with a per-(channel, state) diagonal A ("paper key content" on
  page 1; Mamba1 has no chunk notion, "vLLM Mamba2 SSD kernel warm-up", config/model.py
  section): a_t[c, n] = exp(delta_t[c] * A[c, n]).
* dt preprocessing: dt_bias, dt_softplus and dt_limit as passed by the warm-up call
  (mamba_mixer2.py section of the warm-up page): delta = clamp(softplus(dt + dt_bias)).
* State checkpoints: the state is recorded at the end of every chunk, where chunks never
  span two sequences and every absolute multiple of chunk_size is a cut ("[vLLM] Mamba
  (SSM)", chunk-metadata section: the two guarantees of _compute_chunk_metadata, and
  "why this design", item 3: states saved every chunk_size tokens for prefix caching).
* Decode: one sequential update per token, states gathered through state_indices, rows
  padded with NULL_BLOCK_ID skipped, and the restore checkpoint chosen by
  num_accepted_tokens ("[vLLM] Mamba (SSM)": metadata dataclass, MetadataBuilder init,
  CUDA Graph support section, and "why this design", items 2 and 4).
* Causal depthwise conv1d ahead of the SSD ("vLLM Mamba2 SSD kernel warm-up",
  mamba_mixer2.py section: hidden_states, B and C are taken after a depthwise
  convolution; "vLLM v0.20.0 adds disaggregated serving for hybrid SSM models": the conv
  state of a block is (conv_dim, state_len) or its transpose, state_len 3 in the worked
  example, i.e. a kernel width of 4).  Per channel c with width W and the previous W-1
  inputs kept as the conv state (oldest first):
      out[t, c] = bias[c] + sum_{k=0..W-1} w[c, k] * u[t - (W-1) + k, c]
  where u is the state followed by the new inputs; an optional SiLU v * sigmoid(v)
  follows; the new state is the last W-1 entries of u.
* "all" cache mode (prefix caching, same page: the MetadataBuilder init keeps one state
  index per cache block, and the metadata carries block_idx_first_scheduled_token,
  block_idx_last_computed_token and block_idx_last_scheduled_token).  The pages give the
  names only; the reading used here: a token at absolute position t of its sequence
  belongs to block t // block_size, the state after a block's last token is that block's
  entry, and a partial block's entry holds the state after its last processed token.

Everything is computed in float64 from inputs upcast exactly from their stored dtype.
No blocking, fusion or reordering is applied: tokens are visited one at a time.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "transform_dt", "scan_prefill", "scan_decode", "chunk_metadata", "group_of_head",
    "block_indices", "conv1d_prefill", "conv1d_update",
]


def group_of_head(H: int, G: int) -> np.ndarray:
    """Contiguous head -> group map g(h) = h // (H / G)."""
    if H % G != 0:
        raise ValueError("nheads must be a multiple of ngroups")
    return np.arange(H) // (H // G)


def transform_dt(dt: np.ndarray, dt_bias: Optional[np.ndarray] = None,
                 softplus: bool = False, dt_min: float = 0.0,
                 dt_max: float = math.inf) -> np.ndarray:
    """delta from the raw dt: add dt_bias, apply softplus log(1 + e^v) if requested, then
    clamp to [dt_min, dt_max] (the warm-up call passes dt_bias, dt_softplus=True and
    dt_limit=(0, inf))."""
    v = np.asarray(dt, dtype=np.float64)
    if dt_bias is not None:
        v = v + np.asarray(dt_bias, dtype=np.float64)
    if softplus:
        v = np.logaddexp(0.0, v)
    return np.minimum(np.maximum(v, dt_min), dt_max)


def _step(h: np.ndarray, delta: np.ndarray, A: np.ndarray, x: np.ndarray,
          Bg: np.ndarray, Cg: np.ndarray, D: np.ndarray):
    """One token of the recurrence for all heads.

    h [H, P, N]; delta [H]; A [H] (scalar per head) or [H, N] (diagonal); x [H, P];
    Bg, Cg [H, N] (the group rows each head reads); D [H].  Returns (h_new, y [H, P]).
    """
    if A.ndim == 1:
        decay = np.exp(delta * A)[:, None, None]             # [H, 1, 1]
    else:
        decay = np.exp(delta[:, None] * A)[:, None, :]       # [H, 1, N]
    inject = (delta[:, None] * x)[:, :, None] * Bg[:, None, :]  # delta x B^T  [H, P, N]
    h = decay * h + inject
    y = np.einsum("hpn,hn->hp", h, Cg) + D[:, None] * x
    return h, y


def scan_prefill(x, dt, A, B, C, D, cu_seqlens, chunk_size: int,
                 num_computed=None, initial_states=None, dt_bias=None,
                 dt_softplus: bool = False, dt_min: float = 0.0,
                 dt_max: float = math.inf, block_size: Optional[int] = None):
    """Sequential varlen prefill.

    x [T, H, P]; dt [T, H]; A [H] or [H, N]; B, C [T, G, N]; D [H] or None;
    cu_seqlens [S+1]; num_computed [S] (tokens already processed, default 0);
    initial_states: None, or a list/array of S entries, each None (zero state) or an
    [H, P, N] array.

    Returns a dict with
      y               [T, H, P]           float64
      boundary_states [K, H, P, N]        state after the last token of every chunk, in
                                          chunk order (sequence-major)
      boundary_ends   [K]                 token offset one past each recorded token
      final_states    [S, H, P, N]
      block_states    list of (sequence r, block column b, [H, P, N]) for every new token
                      that closes a cache block (absolute position + 1 a multiple of
                      block_size), in token order; empty unless block_size is given
    """
    x = np.asarray(x, dtype=np.float64)
    T, H, P = x.shape
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    G, N = B.shape[1], B.shape[2]
    A = np.asarray(A, dtype=np.float64)
    D = np.zeros(H) if D is None else np.asarray(D, dtype=np.float64)
    gmap = group_of_head(H, G)
    delta_all = transform_dt(dt, dt_bias, dt_softplus, dt_min, dt_max)
    cu = [int(v) for v in cu_seqlens]
    S = len(cu) - 1
    nc_all = [0] * S if num_computed is None else [int(v) for v in num_computed]

    y = np.zeros((T, H, P))
    boundary, ends, finals, blocks = [], [], [], []
    for r in range(S):
        t0, t1 = cu[r], cu[r + 1]
        h = np.zeros((H, P, N))
        if initial_states is not None and initial_states[r] is not None:
            h = np.array(initial_states[r], dtype=np.float64)
        for t in range(t0, t1):
            h, y[t] = _step(h, delta_all[t], A, x[t], B[t][gmap], C[t][gmap], D)
            absolute = nc_all[r] + (t - t0)          # position of token t in its sequence
            if (absolute + 1) % chunk_size == 0 or t == t1 - 1:
                boundary.append(h.copy())
                ends.append(t + 1)
            if block_size and (absolute + 1) % block_size == 0:
                blocks.append((r, absolute // block_size, h.copy()))
        finals.append(h.copy())
    return {
        "y": y,
        "boundary_states": np.array(boundary).reshape(-1, H, P, N),
        "boundary_ends": np.array(ends, dtype=np.int64),
        "final_states": np.array(finals).reshape(S, H, P, N),
        "block_states": blocks,
    }


def scan_decode(pool, state_indices, num_accepted, x, dt, A, B, C, D,
                null_block_id: int, dt_bias=None, dt_softplus: bool = False,
                dt_min: float = 0.0, dt_max: float = math.inf, rows=None,
                block_idx_last_computed=None, block_idx_last_scheduled=None):
    """Padded, speculative decode step.

    pool [slots, H, P, N] (read only; never modified here); state_indices [B_pad, ntok];
    num_accepted [B_pad] or None (= 1); x [B_pad, ntok, H, P]; dt [B_pad, ntok, H];
    B, C [B_pad, ntok, G, N]; D [H] or None.  ``rows`` restricts the work to a subset of
    rows (independent of each other).

    For a live row r (state_indices[r, 0] != null_block_id), with a = num_accepted[r]:
    the state is read from slot state_indices[r, a-1] before anything is written, then
    for each token j the recurrence advances it, y[r, j] is produced and slot
    state_indices[r, j] receives the state after token j.

    "all" cache mode (block_idx_last_computed and block_idx_last_scheduled given, one
    token per row): state_indices is [B_pad, max_blocks], one entry per cache block; the
    row is padding when its destination entry state_indices[r, last_scheduled[r]] is
    null_block_id; the state is read from state_indices[r, last_computed[r]] and the state
    after the token is written to the destination entry.

    Returns (y, writes): y is a dict row -> [ntok, H, P] for the live rows, writes is a
    dict slot -> [H, P, N] with the state each written slot must hold.
    """
    idx = np.asarray(state_indices)
    all_mode = block_idx_last_scheduled is not None
    B_pad = idx.shape[0]
    ntok = np.asarray(x).shape[1]
    if all_mode and (ntok != 1 or num_accepted is not None):
        raise ValueError("the all cache mode decodes one token per row")
    x = np.asarray(x, dtype=np.float64)
    H, P = x.shape[2], x.shape[3]
    G = B.shape[2]
    A = np.asarray(A, dtype=np.float64)
    D = np.zeros(H) if D is None else np.asarray(D, dtype=np.float64)
    gmap = group_of_head(H, G)
    delta = transform_dt(dt, dt_bias, dt_softplus, dt_min, dt_max)
    y_rows, writes = {}, {}
    for r in (range(B_pad) if rows is None else rows):
        if all_mode:
            dst = [int(idx[r, int(block_idx_last_scheduled[r])])]
            src = int(idx[r, int(block_idx_last_computed[r])]) if dst[0] != null_block_id else 0
        else:
            a = 1 if num_accepted is None else int(num_accepted[r])
            dst = [int(idx[r, j]) for j in range(ntok)]
            src = int(idx[r, a - 1])
        if dst[0] == null_block_id:
            continue
        h = np.array(pool[src], dtype=np.float64)
        ys = np.zeros((ntok, H, P))
        for j in range(ntok):
            Bj = np.asarray(B[r, j], dtype=np.float64)[gmap]
            Cj = np.asarray(C[r, j], dtype=np.float64)[gmap]
            h, ys[j] = _step(h, delta[r, j], A, x[r, j], Bj, Cj, D)
            writes[dst[j]] = h.copy()
        y_rows[r] = ys
    return y_rows, writes


def chunk_metadata(cu_seqlens: Sequence[int], num_computed: Optional[Sequence[int]],
                   chunk_size: int):
    """Brute-force chunk labeler.

    Walks every new token of every sequence at its absolute position p (starting at
    num_computed) and closes a chunk after p when p + 1 is a multiple of chunk_size or p
    is the sequence's last token.  This realises the two guarantees stated for
    _compute_chunk_metadata: a chunk holds tokens of one sequence only, and the state can
    be taken out at every chunk_size-th token.

    Returns (cu_chunk_seqlens [C+1], seq_idx [C], last_chunk_indices [S]) as int32.
    """
    cu = [int(v) for v in cu_seqlens]
    S = len(cu) - 1
    nc = [0] * S if num_computed is None else [int(v) for v in num_computed]
    cuts, owner, last = [0], [], []
    for r in range(S):
        t0, t1 = cu[r], cu[r + 1]
        if t1 <= t0:
            raise ValueError("a sequence without new tokens has no chunk")
        for t in range(t0, t1):
            p = nc[r] + (t - t0)
            if (p + 1) % chunk_size == 0 or t == t1 - 1:
                cuts.append(t + 1)
                owner.append(r)
        last.append(len(owner) - 1)
    return (np.array(cuts, dtype=np.int32), np.array(owner, dtype=np.int32),
            np.array(last, dtype=np.int32))


def block_indices(num_computed: Sequence[int], new_tokens: Sequence[int], block_size: int):
    """Cache-block columns of a batch in the "all" cache mode.

    For a sequence with nc tokens already processed and L new ones, with token t of the
    sequence in block t // block_size:
      first_scheduled = block of the first new token (position nc)
      last_computed   = block of the last processed token (position nc - 1), -1 if nc == 0
      last_scheduled  = block of the last new token (position nc + L - 1)
    Returns the three int32 arrays.
    """
    nc = [int(v) for v in num_computed]
    L = [int(v) for v in new_tokens]
    first = [n // block_size for n in nc]
    last_comp = [(n - 1) // block_size if n > 0 else -1 for n in nc]
    last_sched = [(n + l - 1) // block_size for n, l in zip(nc, L)]
    return (np.array(first, dtype=np.int32), np.array(last_comp, dtype=np.int32),
            np.array(last_sched, dtype=np.int32))


def _conv_window(u: np.ndarray, w: np.ndarray, bias: np.ndarray, activation: bool):
    """Outputs of a causal depthwise conv over u [W-1 + L, D] (state rows first): one row
    per new input, out[i] = bias + sum_k w[:, k] * u[i + k]."""
    W = w.shape[1]
    L = u.shape[0] - (W - 1)
    out = np.zeros((L, u.shape[1]))
    for i in range(L):
        v = bias.copy()
        for k in range(W):
            v = v + w[:, k] * u[i + k]
        if activation:
            v = v / (1.0 + np.exp(-v))
        out[i] = v
    return out


def conv1d_prefill(x, weight, bias, cu_seqlens, conv_states=None,
                   activation: bool = False):
    """Varlen causal depthwise conv1d.

    x [T, D]; weight [D, W]; bias [D] or None; cu_seqlens [S+1]; conv_states: None, or a
    list of S entries, each None (zeros) or a [W-1, D] array (oldest input first).
    Returns (out [T, D], new_states [S, W-1, D]) in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    D, W = w.shape
    b = np.zeros(D) if bias is None else np.asarray(bias, dtype=np.float64)
    cu = [int(v) for v in cu_seqlens]
    out = np.zeros_like(x)
    new_states = []
    for r in range(len(cu) - 1):
        t0, t1 = cu[r], cu[r + 1]
        st = np.zeros((W - 1, D))
        if conv_states is not None and conv_states[r] is not None:
            st = np.asarray(conv_states[r], dtype=np.float64)
        u = np.concatenate([st, x[t0:t1]], axis=0)
        out[t0:t1] = _conv_window(u, w, b, activation)
        new_states.append(u[u.shape[0] - (W - 1):].copy())
    return out, np.array(new_states).reshape(len(cu) - 1, W - 1, D)


def conv1d_update(conv_pool, state_indices, x, weight, bias, null_block_id: int,
                  activation: bool = False):
    """Decode step of the conv: for every row r whose slot state_indices[r] is not
    null_block_id, the row's ntok inputs x[r] [ntok, D] continue the conv state
    conv_pool[slot] [W-1, D] (read, never modified here).  Returns (out, writes): out is a
    dict row -> [ntok, D], writes a dict slot -> the new [W-1, D] state."""
    w = np.asarray(weight, dtype=np.float64)
    D, W = w.shape
    b = np.zeros(D) if bias is None else np.asarray(bias, dtype=np.float64)
    out, writes = {}, {}
    for r in range(len(state_indices)):
        slot = int(state_indices[r])
        if slot == null_block_id:
            continue
        u = np.concatenate([np.asarray(conv_pool[slot], dtype=np.float64),
                            np.asarray(x[r], dtype=np.float64)], axis=0)
        out[r] = _conv_window(u, w, b, activation)
        writes[slot] = u[u.shape[0] - (W - 1):].copy()
    return out, writes
