// ssd_params.h -- kernel parameter blocks and launcher declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd.h"
#include "ssd_device.h"
#include "ssd_plan.h"

namespace ssd {

// Everything the prefill kernels read, resolved from ssd_prefill_args and the plan.
struct PrefillParams {
  int T, H, P, G, N, S, C, cs;
  const void* x;  int64_t x_st;
  const void* dt; int64_t dt_st;
  const void* B;
  const void* Cm; int64_t bc_st;
  void* y;        int64_t y_st;
  const float* A;
  const float* D;
  DtPrep prep;
  const int* cu_seqlens;
  const int* cu_chunk;
  const int* seq_idx;
  const int* last_chunk;
  void* pool; int64_t slot_stride; int num_slots;
  int pool_kind;       // dtype of the pool states: 0 fp32, 1 bf16, 2 fp16 (state_dtype)
  const int* state_idx;
  const int* has_init;
  int write_final;
  int block_size;      // > 0: the all cache mode (state_idx is [S, idx_stride])
  int idx_stride;
  const int* num_computed;
  const int* blk_last_comp;
  const int* blk_last_sched;
  float* states;       // [C, H, P, N] chunk_states_out (NULL: not written)
  void* cbw;           // workspace, input dtype: C.B^T fragments per chunk and group
  void* btw;           // workspace, input dtype: B^T fragments per chunk and group
  float* dcw;          // workspace [C, H, 2, cs]: cumsum of delta*A, then delta
  void* cfw;           // workspace, input dtype: C fragments per chunk and group
  int* seq_ord;        // workspace [S]: sequences in march dispatch order
  int* chain_flag;     // workspace [C, H, kChainWaves]: chain publication flags (NULL: march)
  int* items;          // workspace [chain_grid]: the chain kernel's (chunk * H + head) per
                       // workgroup, -1 for none (NULL: chunks in index order)
  int chain_grid;      // workgroups of the chain kernel
  float* hring;        // workspace [S, H, 2, P, N] when states is NULL: published states
  int* blk_slot;       // workspace [C], all cache mode: pool slot of each chunk's end state
                       // (-1: none), set by k_chunk_prep; NULL when the mode is off
  int* flag;
  float* dA_cumsum_out;
  float* cb_out;
  float* local_states_out;
};

// Pool entries of a sequence (the chunked kernels and the diagonal scan share these).
// state_idx is [S, idx_stride]: one slot per sequence (idx_stride 1, column 0), or in the
// all cache mode one entry per cache block of block_size tokens (block b: tokens
// [b*block_size, (b+1)*block_size) of the sequence).

// Slot of entry `col` of sequence r, or -1 (SSD_DEVERR_SLOT_RANGE raised if `report`)
// when the column or the slot is out of range.
__device__ __forceinline__ int pool_slot(const PrefillParams& p, int r, int col, bool report) {
  int slot = -1;
  if (col >= 0 && col < p.idx_stride) slot = p.state_idx[int64_t(r) * p.idx_stride + col];
  if (slot < 0 || slot >= p.num_slots) {
    if (report) raise_flag(p.flag, SSD_DEVERR_SLOT_RANGE);
    return -1;
  }
  return slot;
}

// The all cache mode's entry for the state at the end of chunk [cs0, cs1) of sequence r
// (first token t0): column e / block_size - 1 when the chunk ends at an absolute position
// e that closes a block, else -1.  A block end strictly inside the chunk means the chunk
// metadata was built for another num_computed: SSD_DEVERR_CHUNK_RANGE if `report`.
__device__ __forceinline__ int block_end_col(const PrefillParams& p, int r, int t0, int cs0,
                                             int cs1, bool report) {
  if (p.block_size <= 0) return -1;
  // absolute positions fit in int32 (the chunk-metadata builder rejects larger ones)
  const int64_t a0 = int64_t(p.num_computed[r]) + (cs0 - t0), a1 = a0 + (cs1 - cs0);
  const uint32_t bs = uint32_t(p.block_size), u0 = uint32_t(a0), u1 = uint32_t(a1);
  if (a0 < 0 || a1 > INT32_MAX || (u1 - 1) / bs != u0 / bs) {
    if (report) raise_flag(p.flag, SSD_DEVERR_CHUNK_RANGE);
    return -1;
  }
  return u1 % bs == 0 ? int(u1 / bs) - 1 : -1;
}

// Source and final pool slots of sequence r (-1: none): the sequence's slot, or in the all
// cache mode the entries block_idx_last_computed (read only with an initial state) and
// block_idx_last_scheduled (written only with write_final).
struct SeqSlots { int src, fin; };
__device__ __forceinline__ SeqSlots seq_slots(const PrefillParams& p, int r, bool need_src,
                                              bool need_fin, bool report) {
  SeqSlots s{-1, -1};
  if (!p.pool || !p.state_idx || !(need_src || need_fin)) return s;
  if (p.block_size <= 0) {
    const int slot = pool_slot(p, r, 0, report);
    s.src = need_src ? slot : -1;
    s.fin = need_fin ? slot : -1;
    return s;
  }
  if (need_src && p.has_init && p.has_init[r]) s.src = pool_slot(p, r, p.blk_last_comp[r], report);
  if (need_fin && p.write_final) s.fin = pool_slot(p, r, p.blk_last_sched[r], report);
  return s;
}

struct DecodeParams {
  int B_pad, ntok, H, P, G, N;
  int diag;            // SSD_A_DIAG: A is [H, N] (Mamba1, P == 1, G == 1)
  const void* x;
  const void* dt;
  const void* B;
  const void* Cm;
  void* y;
  const float* A;
  const float* D;
  DtPrep prep;
  void* pool; int64_t slot_stride; int num_slots;
  int pool_kind;       // dtype of the pool states: 0 fp32, 1 bf16, 2 fp16 (state_dtype)
  const int* idx;
  const int* num_acc;
  int null_id;
  int* flag;
  int idx_stride;      // > 0: the all cache mode (idx is [B_pad, idx_stride], ntok == 1)
  const int* blk_last_comp;
  const int* blk_last_sched;
};

// `events` (may be NULL): hipEvent_t handles recorded before each launch and after the
// last one (the timing hook of the C ABI).
hipError_t launch_chunked_prefill(int variant, const PrefillParams& p, hipStream_t s,
                                  void* const* events);
// The sequential scan of a one-element head: scalar_a selects A [H] (head_dim 1) over the
// per-(channel, state) A [H, N].
hipError_t launch_diag_prefill(int in_dtype, bool scalar_a, const PrefillParams& p, hipStream_t s,
                               void* const* events);
// True when the sequential scan of S sequences runs the grid of 64- and 32-channel
// workgroups (k_diag_scan_mixed) on the current device, false for k_diag_scan.
bool diag_mixed_grid(bool scalar_a, int S, int H, int G, int N);
hipError_t launch_state_update(int in_dtype, const DecodeParams& p, hipStream_t s,
                               void* const* events);

// SSD_DEBUG: the distinct-slot checks (ssd_debug.hip), launched before a call's kernels.
bool debug_checks_enabled();
hipError_t launch_prefill_slot_check(const PrefillParams& p, hipStream_t s);
hipError_t launch_decode_slot_check(const DecodeParams& p, hipStream_t s);

inline void record_event(void* const* events, int i, hipStream_t s) {
  if (events && events[i]) (void)hipEventRecord(static_cast<hipEvent_t>(events[i]), s);
}

// Dynamic LDS of the decode kernel for these sizes (host checks it against the limit).
inline size_t decode_lds_bytes(int ntok, int P, int N) {
  return size_t(ntok) * (2 * P + 2 * N + 1) * sizeof(float);
}

}  // namespace ssd
