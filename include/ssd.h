/*
 * ssd.h -- C ABI of the MI355X (gfx950) Mamba2 SSD selective-state-space scan library.
 *
 * Three calls make up the path:
 *   ssd_build_chunk_metadata  host, integer: split a varlen prefill batch into chunks;
 *   ssd_prefill               device: chunked varlen prefill with initial states gathered
 *                             from a state pool and the state written at every chunk end;
 *   ssd_state_update          device: padded single-token / speculative decode update.
 * and two more the step before it needs (the causal depthwise conv1d whose outputs are
 * the scan's x, B and C): ssd_conv1d_prefill and ssd_conv1d_update.
 *
 * The recurrence (per head h, state in R^{P x N}):
 *     h_t = exp(delta_t * A_h) * h_{t-1} + delta_t * x_t B_t^T,   y_t = h_t C_t + D_h x_t
 * is the selective SSM whose Delta, B and C depend on the input ("[vLLM] Mamba (SSM):
 * linear-time sequence modeling", intro and paper key content).  Heads map onto B/C
 * groups in contiguous blocks, g(h) = h / (H / G).
 *
 * Conventions shared by every call:
 *   - Sizes and counts are int32; strides are in ELEMENTS of the tensor's dtype.
 *   - "device" pointers are HIP device (or managed) memory; "host" pointers are ordinary
 *     CPU memory.  The caller owns every buffer.  The library allocates nothing, keeps no
 *     pointer after a call returns, never synchronises and launches only on `stream`.
 *   - Every argument check that does not need device data runs before the first launch:
 *     a call that returns an error launched nothing.  Checks that need device data
 *     (index ranges, metadata consistency) run in the kernels: the offending item is
 *     skipped (nothing of it is written) and *device_error_flag, when non-NULL, is set to
 *     a nonzero SSD_DEVERR_* bit mask (the flag is only ever OR-ed, never cleared).
 *   - No global mutable state: calls on different streams may run concurrently as long
 *     as they do not write the same memory.
 *   - The pool is updated in place: two sequences of one prefill, or two live rows of one
 *     decode, must not touch the same pool slot (a race otherwise).  With the environment
 *     variable SSD_DEBUG set (to anything but "0") each call first launches a check kernel
 *     that raises SSD_DEVERR_DUPLICATE_SLOT when they do (O(n^2) in the entries touched;
 *     not counted by ssd_prefill_kernel_count, not timed by profile_events).
 */
#ifndef SSD_MI355X_H
#define SSD_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 3

typedef enum ssd_status {
  SSD_OK = 0,
  SSD_ERR_NULL_POINTER = 1,  /* a required pointer is NULL                              */
  SSD_ERR_BAD_SHAPE = 2,     /* a size or stride is out of range / inconsistent         */
  SSD_ERR_BAD_METADATA = 3,  /* host metadata inputs are inconsistent                   */
  SSD_ERR_UNSUPPORTED = 4,   /* (dtype, head_dim, dstate, chunk_size) not instantiated  */
  SSD_ERR_CAPACITY = 5,      /* an output array is too small; the required size is
                                reported through the *_out count argument              */
  SSD_ERR_WORKSPACE = 6,     /* workspace NULL or smaller than ssd_prefill_workspace_size */
  SSD_ERR_HIP = 7            /* a HIP launch failed                                     */
} ssd_status;

/* device-side error bits OR-ed into *device_error_flag */
#define SSD_DEVERR_CHUNK_RANGE 1   /* a chunk is empty, longer than chunk_size or leaves
                                      its sequence                                     */
#define SSD_DEVERR_SLOT_RANGE 2    /* a state index is outside [0, num_slots)           */
#define SSD_DEVERR_ACCEPTED 4      /* num_accepted_tokens outside [1, ntok]            */
#define SSD_DEVERR_CHAIN_WAIT 8    /* a chunk could not take over its predecessor's state:
                                      it waited about a second (only inconsistent chunk
                                      metadata leaves a predecessor unprocessed), or the
                                      state was left in the L2 of another XCD than the one
                                      workgroup dispatch placed the chunk on; the outputs
                                      of that sequence are invalid                       */
#define SSD_DEVERR_DUPLICATE_SLOT 16 /* two sequences (prefill) or two decode rows touch
                                      the same pool slot; only checked when the
                                      environment variable SSD_DEBUG is set (not "0"),
                                      by an extra kernel each call launches first        */

typedef enum ssd_dtype { SSD_F32 = 0, SSD_BF16 = 1, SSD_F16 = 2 } ssd_dtype;

typedef enum ssd_a_kind {
  SSD_A_SCALAR = 0,  /* Mamba2: A[H], one decay per head                                 */
  SSD_A_DIAG = 1     /* Mamba1: A[H, N], one decay per (channel, state); requires P == 1 */
} ssd_a_kind;

/* A hipStream_t passed as an opaque pointer (NULL = the null stream). */
typedef void* ssd_stream_t;

/* ---------------------------------------------------------------------------------------
 * Library information
 * ------------------------------------------------------------------------------------- */
int ssd_abi_version(void);
const char* ssd_status_string(ssd_status status); /* static string, never NULL */

/* ---------------------------------------------------------------------------------------
 * Chunk metadata (host, integer, bit-exact)
 *
 * Defined by the chunk-metadata section of "[vLLM] Mamba (SSM): linear-time sequence
 * modeling" (_compute_chunk_metadata): every chunk holds tokens of ONE sequence, and a
 * chunk ends at every absolute multiple of chunk_size so the state can be taken out
 * there.  A resumed sequence whose num_computed is not a multiple of chunk_size first
 * finishes the open chunk with min(cdiv(nc, cs) * cs - nc, new_tokens) tokens; the rest
 * is cut into chunks of min(cs, remaining) tokens.  The page's listing stops after the
 * partial-chunk branch; the rest (full chunks, then the tail) is the plain reading of its
 * two stated guarantees.  The single-chunk case matches the warm-up inputs of "vLLM Mamba2
 * SSD kernel warm-up" (mamba_mixer2.py section): cu_seqlens=[0,cs] gives
 * cu_chunk_seqlens=[0,cs], seq_idx=[0], last_chunk_indices=[0].
 *
 *   num_seqs            S >= 0
 *   cu_seqlens          host int32 [S+1], cu_seqlens[0] == 0, strictly increasing (every
 *                       sequence has >= 1 new token)
 *   num_computed        host int32 [S] tokens already processed per sequence (>= 0), or
 *                       NULL for all zero
 *   chunk_size          > 0
 *   capacity            entries available in seq_idx (cu_chunk_seqlens must hold
 *                       capacity + 1 entries); last_chunk_indices must hold S entries
 *   cu_chunk_seqlens    host int32 [C+1] out: token offset of every chunk start, then T
 *   seq_idx             host int32 [C]   out: sequence of every chunk
 *   last_chunk_indices  host int32 [S]   out: index of every sequence's last chunk
 *   num_chunks_out      host int32       out: C (also on SSD_ERR_CAPACITY)
 *
 * Errors: SSD_ERR_NULL_POINTER, SSD_ERR_BAD_SHAPE (S < 0, chunk_size <= 0),
 * SSD_ERR_BAD_METADATA (cu_seqlens[0] != 0, a sequence with < 1 token, num_computed < 0,
 * num_computed + new tokens beyond INT32_MAX, an int32 overflow), SSD_ERR_CAPACITY
 * (C > capacity; nothing but *num_chunks_out is written).
 * ------------------------------------------------------------------------------------- */
ssd_status ssd_chunk_metadata_count(int32_t num_seqs, const int32_t* cu_seqlens,
                                    const int32_t* num_computed, int32_t chunk_size,
                                    int32_t* num_chunks_out);
ssd_status ssd_build_chunk_metadata(int32_t num_seqs, const int32_t* cu_seqlens,
                                    const int32_t* num_computed, int32_t chunk_size,
                                    int32_t capacity, int32_t* cu_chunk_seqlens,
                                    int32_t* seq_idx, int32_t* last_chunk_indices,
                                    int32_t* num_chunks_out);

/* ---------------------------------------------------------------------------------------
 * Prefill
 *
 * The argument set follows the varlen SSD call made by the warm-up code of "vLLM Mamba2
 * SSD kernel warm-up" (mamba_mixer2.py section): x, dt, A, B, C, chunk_size, cu_seqlens,
 * cu_chunk_seqlens, last_chunk_indices, seq_idx, out, D, dt_bias, initial_states,
 * dt_softplus, dt_limit and an fp32 state dtype.  Initial states are gathered from a state
 * pool laid out [slots, H, P, N] (the SSM block shape (num_heads, head_dim, state_size) of
 * "vLLM v0.20.0 adds disaggregated serving for hybrid SSM models"), selected per sequence
 * by state_indices and has_initial_state ("[vLLM] Mamba (SSM)", metadata dataclass:
 * has_initial_states_p, state_indices_tensor_p).  The state at the end of every chunk is
 * written out for prefix caching ("why this design", item 3).
 *
 * Computes, for every sequence r (tokens [cu_seqlens[r], cu_seqlens[r+1])):
 *   h = has_initial_state[r] ? pool[state_indices[r]] : 0
 *   for each token t, head h:  delta = clamp(softplus?(dt[t,h] + dt_bias[h]), dt_min, dt_max)
 *       state = exp(delta*A) state + delta x[t,h,:] B[t,g,:]^T;  y[t,h,:] = state C[t,g,:] + D x
 *   chunk_states_out[k] = state after the last token of chunk k (every chunk)
 *   if write_final_to_pool: pool[state_indices[r]] = state after the sequence's last token
 * The pool slots are read before any is written (a sequence may resume from, and write
 * back to, the same slot).  state_indices of different sequences must be distinct.
 * ------------------------------------------------------------------------------------- */
typedef struct ssd_prefill_args {
  /* sizes */
  int32_t T;            /* total tokens (sum of sequence lengths)                      */
  int32_t H;            /* heads (SSD_A_SCALAR) or channels d_inner (SSD_A_DIAG)        */
  int32_t P;            /* head_dim (1 for SSD_A_DIAG)                                  */
  int32_t G;            /* B/C groups; H % G == 0 (1 for SSD_A_DIAG)                    */
  int32_t N;            /* dstate                                                       */
  int32_t chunk_size;   /* cs                                                           */
  int32_t num_seqs;     /* S                                                            */
  int32_t num_chunks;   /* C, as returned by ssd_build_chunk_metadata                   */
  int32_t in_dtype;     /* ssd_dtype of x, dt, B, C and y: SSD_F32 or SSD_BF16            */
  int32_t a_kind;       /* ssd_a_kind                                                   */

  /* token tensors (device).  Within one token the layout is contiguous ([H,P] / [H] /
   * [G,N]); the *_stride_t arguments give the distance between consecutive tokens, so x,
   * B and C may be views into one projection buffer. */
  const void* x;  int64_t x_stride_t;   /* [T, H, P], stride >= H*P                       */
  const void* dt; int64_t dt_stride_t;  /* [T, H],    stride >= H                         */
  const void* B;                        /* [T, G, N]                                      */
  const void* C;  int64_t bc_stride_t;  /* [T, G, N], stride >= G*N (shared by B and C)    */
  void* y;        int64_t y_stride_t;   /* [T, H, P] out, in_dtype, stride >= H*P         */

  /* parameters (device, fp32) */
  const float* A;        /* [H] (SSD_A_SCALAR) or [H, N] (SSD_A_DIAG); not NULL         */
  const float* D;        /* [H] skip connection, NULL = 0                                */
  const float* dt_bias;  /* [H], NULL = 0                                                */
  int32_t dt_softplus;   /* 0/1: apply log(1 + e^v) after adding dt_bias                 */
  float dt_min, dt_max;  /* clamp applied last; (0, +inf) is the usual limit             */

  /* chunk metadata (device int32), from ssd_build_chunk_metadata */
  const int32_t* cu_seqlens;         /* [S+1] */
  const int32_t* cu_chunk_seqlens;   /* [C+1] */
  const int32_t* seq_idx;            /* [C]   */
  const int32_t* last_chunk_indices; /* [S]   */

  /* state pool (device, fp32, [num_slots, H, P, N] with slot_stride elements between
   * slots, slot_stride >= H*P*N), in state_dtype.  May be NULL when no sequence has an
   * initial state and write_final_to_pool == 0. */
  void* state_pool;
  int64_t slot_stride;
  int32_t num_slots;
  const int32_t* state_indices;      /* [S] slot per sequence (device); NULL only without a pool */
  const int32_t* has_initial_state;  /* [S] 0/1 (device); NULL = no initial states          */
  int32_t write_final_to_pool;       /* 0/1                                               */

  /* outputs (device) */
  float* chunk_states_out;   /* [C, H, P, N] fp32 state at the end of every chunk; NULL =
                                not wanted (a workspace holds them instead)              */
  int32_t* device_error_flag;/* NULL or an int32 that receives SSD_DEVERR_* bits         */

  /* optional per-step outputs (device, NULL = not wanted; SSD_A_SCALAR only) */
  float* dA_cumsum_out;      /* [H, T] fp32: inclusive within-chunk cumsum of delta*A     */
  float* cb_out;             /* [C, G, cs, cs] fp32: C_l . B_s for s <= l < chunk length,
                                other entries untouched                                   */
  float* chunk_local_states_out; /* [C, H, P, N] fp32: the state each chunk produces from a
                                zero state (before the inter-chunk pass)                  */

  /* optional timing hook: NULL, or SSD_PREFILL_MAX_KERNELS + 1 hipEvent_t handles (created
   * by the caller) that the call records on `stream` before each of its kernels and after
   * the last one; entries past the kernels this call launches are not touched.  The number
   * of kernels launched is reported by ssd_prefill_kernel_count. */
  void* const* profile_events;

  /* ssd_dtype of state_pool: SSD_F32 (0, so a zero-initialised struct keeps fp32), SSD_BF16
   * or SSD_F16 (a bf16 or IEEE fp16 pool, the reduced-precision SSM state dtypes of "vLLM
   * Mamba2 SSD kernel warm-up", mamba_mixer2.py section): states are read from and written
   * to the pool in that dtype (round to nearest even; an fp16 state beyond 65504 in
   * magnitude becomes infinite) and carried in fp32 everywhere else; chunk_states_out stays
   * fp32.  Any other value: SSD_ERR_BAD_SHAPE. */
  int32_t state_dtype;

  /* "all" cache mode: prefix caching with one state entry per cache block ("[vLLM] Mamba
   * (SSM)": the MetadataBuilder init sizes the decode index tensor by the maximum number
   * of blocks in this mode, and the metadata carries block_idx_first_scheduled_token,
   * block_idx_last_computed_token and block_idx_last_scheduled_token).  block_size == 0
   * keeps one slot per sequence as described above.  With block_size > 0 (a multiple of
   * chunk_size; either a_kind):
   *   - state_indices is [S, idx_stride]: entry (r, b) is the pool slot of cache block b of
   *     sequence r, the block of the sequence's tokens [b*block_size, (b+1)*block_size);
   *   - the initial state (has_initial_state[r]) is read from entry
   *     (r, block_idx_last_computed[r]);
   *   - a chunk whose end lies at absolute position e of its sequence (num_computed[r]
   *     plus the sequence's new tokens up to the chunk end) with e % block_size == 0 writes
   *     its end state to entry (r, e / block_size - 1);
   *   - with write_final_to_pool the final state goes to entry
   *     (r, block_idx_last_scheduled[r]);
   *   - block_idx_first_scheduled_token is not an input: it is num_computed / block_size,
   *     the entry of the first block end above.
   * A partial block's entry holds the state after its last processed token, so a sequence
   * may resume from the entry it then overwrites.  Entries written by one sequence must not
   * be read or written by another.  A column or slot out of range skips that read or write
   * and raises SSD_DEVERR_SLOT_RANGE; a block end falling inside a chunk (num_computed not
   * the value the chunk metadata was built with) raises SSD_DEVERR_CHUNK_RANGE. */
  int32_t block_size;
  int32_t idx_stride;                       /* row stride of state_indices, >= 1      */
  const int32_t* num_computed;              /* [S] (device) tokens processed before    */
  const int32_t* block_idx_last_computed;   /* [S] (device) entry of the initial state */
  const int32_t* block_idx_last_scheduled;  /* [S] (device) entry of the final state   */
} ssd_prefill_args;

#define SSD_PREFILL_MAX_KERNELS 2

/* Number of kernels ssd_prefill launches for these arguments (2 for SSD_A_SCALAR, 1 for
 * SSD_A_DIAG, 0 for an empty batch) and, when `names` is not NULL, a static name for each
 * kernel in launch order (names must hold SSD_PREFILL_MAX_KERNELS entries).  The diagonal
 * scan's grid, and so its kernel's name, depends on the batch and on the current device's
 * compute-unit count (256 when no device is present). */
ssd_status ssd_prefill_kernel_count(const ssd_prefill_args* args, int32_t* count,
                                    const char** names);

/* Bytes of device workspace ssd_prefill needs for these arguments (0 is possible).  The
 * workspace must be 256-byte aligned and must not alias any argument.  It holds no state
 * between calls.  Errors: as ssd_prefill's host checks. */
ssd_status ssd_prefill_workspace_size(const ssd_prefill_args* args, size_t* bytes);

/* Run the prefill on `stream`.  workspace: device memory of >= the reported size (may be
 * NULL when that size is 0).  Errors: SSD_ERR_NULL_POINTER, SSD_ERR_BAD_SHAPE,
 * SSD_ERR_UNSUPPORTED, SSD_ERR_WORKSPACE, SSD_ERR_HIP.  T == 0 (with S == 0) is a no-op. */
ssd_status ssd_prefill(const ssd_prefill_args* args, void* workspace,
                       size_t workspace_bytes, ssd_stream_t stream);

/* Allocation-free variant of ssd_prefill, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same kernels run with their workspace in a static device array of
 * SSD_NOALLOC_SCRATCH_BYTES (256 MiB) that the library holds on every GPU it runs on until
 * the process ends; the call itself allocates and frees nothing.  The caller still passes
 * every input and output.  Every ssd_prefill_noalloc call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (different streams, or host threads) race
 * and give undefined results; calls in stream order are safe (each call's kernels set up
 * everything they read from the array, nothing needs clearing in between).
 * Errors: as ssd_prefill, plus SSD_ERR_WORKSPACE when the workspace these arguments need
 * (ssd_prefill_workspace_size) exceeds SSD_NOALLOC_SCRATCH_BYTES, and SSD_ERR_HIP when the
 * array's device address cannot be obtained. */
#define SSD_NOALLOC_SCRATCH_BYTES (256u << 20)
ssd_status ssd_prefill_noalloc(const ssd_prefill_args* args, ssd_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Decode state update
 *
 * One decode step for a padded, uniform batch ("[vLLM] Mamba (SSM)": decode metadata,
 * MetadataBuilder init with a (max batch, 1 + num_spec_tokens) index tensor, and the CUDA
 * Graph section, which pads the rows past the live ones with NULL_BLOCK_ID so one graph
 * serves every batch size).  Every row carries ntok = 1 + num_spec_tokens tokens.
 *
 * For every row r with state_indices[r, 0] != null_block_id (other rows are skipped: no
 * state read, no write, y untouched):
 *   a = num_accepted_tokens[r] (1 if the pointer is NULL)
 *   state = pool[state_indices[r, a-1]]        (read before any slot is written; this is
 *                                               the restore from the right checkpoint of
 *                                               "why this design", item 4)
 *   for j in 0..ntok-1:  advance state by token (r, j); y[r, j] = state C + D x;
 *                        pool[state_indices[r, j]] = state
 * Slot indices of live rows must be distinct across rows (a row may read the slot it
 * writes).  All ntok outputs are produced: acceptance is decided after this step.
 * With SSD_A_DIAG the same step runs the Mamba1 recurrence of the diagonal scan above
 * (decay exp(delta[c] A[c, n]) per channel c and state n; H channels, P == 1, G == 1,
 * N == 16), the single-token counterpart of the Mamba1 prefill.
 * ------------------------------------------------------------------------------------- */
typedef struct ssd_decode_args {
  int32_t B_pad;        /* rows, including padding rows                                 */
  int32_t ntok;         /* tokens per row = 1 + speculative tokens, >= 1                */
  int32_t H, P, G, N;
  int32_t in_dtype;     /* ssd_dtype of x, dt, B, C and y: SSD_F32 or SSD_BF16            */
  int32_t a_kind;       /* SSD_A_SCALAR, or SSD_A_DIAG (Mamba1: P == 1, G == 1, N == 16) */

  /* token tensors (device, contiguous) */
  const void* x;        /* [B_pad, ntok, H, P] */
  const void* dt;       /* [B_pad, ntok, H]    */
  const void* B;        /* [B_pad, ntok, G, N] */
  const void* C;        /* [B_pad, ntok, G, N] */
  void* y;              /* [B_pad, ntok, H, P] out */

  const float* A;       /* [H], or [H, N] for SSD_A_DIAG */
  const float* D;       /* [H] or NULL */
  const float* dt_bias; /* [H] or NULL */
  int32_t dt_softplus;
  float dt_min, dt_max;

  void* state_pool;     /* [num_slots, H, P, N] in state_dtype, slot_stride >= H*P*N */
  int64_t slot_stride;
  int32_t num_slots;
  const int32_t* state_indices;       /* [B_pad, ntok] (device) */
  const int32_t* num_accepted_tokens; /* [B_pad] (device) or NULL */
  int32_t null_block_id;
  int32_t* device_error_flag;         /* NULL or an int32 receiving SSD_DEVERR_* bits */
  void* const* profile_events;        /* NULL or 2 hipEvent_t recorded before and after
                                         the update kernel (timing hook)              */
  int32_t state_dtype;                /* ssd_dtype of state_pool: SSD_F32 (0), SSD_BF16
                                         or SSD_F16 (a 2-byte pool with a dense A needs
                                         slot_stride % 8 == 0); the state is carried in
                                         fp32 inside the step                          */

  /* "all" cache mode (one state entry per cache block, as for the prefill): idx_stride ==
   * 0 keeps state_indices [B_pad, ntok] as described above.  With idx_stride > 0,
   * state_indices is [B_pad, idx_stride], ntok must be 1 and num_accepted_tokens NULL; a
   * row is padding when its destination entry state_indices[r, block_idx_last_scheduled[r]]
   * is null_block_id; otherwise the state is read from entry
   * (r, block_idx_last_computed[r]) and the state after the token is written to the
   * destination entry.  A column out of range skips the row and raises
   * SSD_DEVERR_SLOT_RANGE. */
  int32_t idx_stride;
  const int32_t* block_idx_last_computed;   /* [B_pad] (device) */
  const int32_t* block_idx_last_scheduled;  /* [B_pad] (device) */
} ssd_decode_args;

/* Errors: SSD_ERR_NULL_POINTER (also a NULL block index array in the all cache mode),
 * SSD_ERR_BAD_SHAPE (also an unknown a_kind, SSD_A_DIAG with P != 1 or G != 1, or the all
 * cache mode with ntok != 1 or num_accepted_tokens set), SSD_ERR_UNSUPPORTED (N, ntok or
 * P*N outside the instantiated range; state_pool not 16-byte aligned or slot_stride not a
 * multiple of 4, or of 8 for a bf16 or fp16 pool with SSD_A_SCALAR), SSD_ERR_HIP.
 * B_pad == 0 is a no-op. */
ssd_status ssd_state_update(const ssd_decode_args* args, ssd_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Causal depthwise conv1d (the convolution whose outputs the SSD takes as x, B and C)
 *
 * "vLLM Mamba2 SSD kernel warm-up" (mamba_mixer2.py section) takes hidden_states, B and C
 * after a depthwise convolution; "vLLM v0.20.0 adds disaggregated serving for hybrid SSM
 * models" keeps one conv state per cache block, (conv_dim, state_len) or its transpose,
 * with state_len 3 in its worked example ([num_blocks, 3, 3072]).  Per channel c of D, a
 * width-W causal filter runs over the W-1 carried inputs followed by the new ones:
 *   out[t, c] = act(bias[c] + sum_{k=0..W-1} weight[c, k] * u[t - (W-1) + k, c])
 * (weight[c, W-1] multiplies the newest input; act is the identity or SiLU v*sigmoid(v)),
 * and the conv state becomes the last W-1 inputs of u (the old state shifted left when a
 * sequence has fewer than W-1 new inputs).  W == 4 is the instantiated width.
 *
 * Conv state pool: element (slot, k, c) of a [num_slots] pool with slot_stride elements
 * between slots, k = 0 the oldest input, in in_dtype, laid out
 *   SSD_CONV_LAYOUT_SD: [slot][k][c]  (slot_stride >= (W-1)*D, the printed block shape)
 *   SSD_CONV_LAYOUT_DS: [slot][c][k]  (slot_stride >= D*(W-1), the per-channel layout)
 * ------------------------------------------------------------------------------------- */
#define SSD_CONV_LAYOUT_SD 0
#define SSD_CONV_LAYOUT_DS 1
#define SSD_CONV_MAX_KERNELS 2

typedef struct ssd_conv1d_args {
  int32_t T;            /* total tokens                                                 */
  int32_t D;            /* channels (conv_dim), a multiple of 8                         */
  int32_t W;            /* kernel width                                                 */
  int32_t num_seqs;     /* S                                                            */
  int32_t num_chunks;   /* C of the chunk metadata (ssd_build_chunk_metadata, any
                           chunk_size): the unit of work, never two sequences           */
  int32_t in_dtype;     /* ssd_dtype of x, out and the conv state: SSD_F32 or SSD_BF16    */
  const void* x;   int64_t x_stride_t;    /* [T, D] (device), stride >= D               */
  void* out;       int64_t out_stride_t;  /* [T, D] out (device), stride >= D           */
  const float* weight;  /* [D, W] (device, fp32)                                          */
  const float* bias;    /* [D] (device, fp32) or NULL = 0                                 */
  int32_t activation;   /* 0: none, 1: SiLU                                               */
  const int32_t* cu_seqlens;        /* [S+1] (device) */
  const int32_t* cu_chunk_seqlens;  /* [C+1] (device) */
  const int32_t* seq_idx;           /* [C]   (device) */
  void* conv_states;    /* pool (device) or NULL: zero initial states, nothing written     */
  int64_t slot_stride;
  int32_t num_slots;
  int32_t state_layout;               /* SSD_CONV_LAYOUT_*                                */
  const int32_t* state_indices;       /* [S] slot per sequence (device); NULL only without
                                         a pool                                           */
  const int32_t* has_initial_state;   /* [S] 0/1 (device) or NULL = none                  */
  int32_t* device_error_flag;         /* NULL or an int32 receiving SSD_DEVERR_* bits     */
  void* const* profile_events;        /* NULL or SSD_CONV_MAX_KERNELS + 1 hipEvent_t,
                                         recorded before each kernel and after the last */
} ssd_conv1d_args;

/* Varlen prefill of the conv: out for every token; with a pool, each sequence's state is
 * read (has_initial_state) and then replaced by its last W-1 inputs, in place.  Two
 * kernels: the outputs, then the state writes (so every read of an old state precedes
 * every write).  state_indices of different sequences must be distinct.  Errors:
 * SSD_ERR_NULL_POINTER, SSD_ERR_BAD_SHAPE, SSD_ERR_UNSUPPORTED (W != 4, D % 8, pointers
 * not 16-byte aligned, strides not multiples of 8 elements, or (T/8 + 1) rows of x or out
 * spanning 2 GiB or more), SSD_ERR_HIP.  Device
 * checks: a bad chunk raises SSD_DEVERR_CHUNK_RANGE, a slot out of range
 * SSD_DEVERR_SLOT_RANGE (that sequence's state is neither read nor written).  S == 0 is a
 * no-op. */
ssd_status ssd_conv1d_prefill(const ssd_conv1d_args* args, ssd_stream_t stream);

typedef struct ssd_conv1d_update_args {
  int32_t B_pad;        /* rows, including padding rows                                 */
  int32_t ntok;         /* inputs per row, 1..16, processed in order                    */
  int32_t D, W;
  int32_t in_dtype;
  const void* x;        /* [B_pad, ntok, D] (device, contiguous)                          */
  void* out;            /* [B_pad, ntok, D] out                                           */
  const float* weight;  /* [D, W] fp32                                                    */
  const float* bias;    /* [D] fp32 or NULL                                               */
  int32_t activation;
  void* conv_states;    /* pool (device), as for the prefill                              */
  int64_t slot_stride;
  int32_t num_slots;
  int32_t state_layout;
  const int32_t* state_indices;  /* [B_pad] (device); rows whose entry is null_block_id are
                                    padding: nothing read or written                      */
  int32_t null_block_id;
  int32_t* device_error_flag;
  void* const* profile_events;   /* NULL or 2 hipEvent_t around the kernel                */
} ssd_conv1d_update_args;

/* Decode step of the conv: each live row's ntok inputs continue its slot's state, which is
 * then replaced in place.  Slots of live rows must be distinct.  Errors as for the
 * prefill (also ntok outside 1..16: SSD_ERR_UNSUPPORTED); a slot out of range skips the
 * row and raises SSD_DEVERR_SLOT_RANGE.  B_pad == 0 is a no-op. */
ssd_status ssd_conv1d_update(const ssd_conv1d_update_args* args, ssd_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SSD_MI355X_H */
