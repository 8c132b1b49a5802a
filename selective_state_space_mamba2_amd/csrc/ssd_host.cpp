// ssd_host.cpp -- host half of the C ABI: status strings, the chunk-metadata builder,
// argument validation and workspace planning.  Plain C++; needs no GPU.
#include <cmath>
#include <cstdint>
#include <limits>

#include "ssd.h"
#include "ssd_plan.h"

namespace ssd {

// Chunked-prefill instantiations: (dtype, head_dim, dstate, chunk_size).  The kernels'
// launch table in ssd_prefill.hip lists the same shapes in the same order.
const ChunkedShape kChunkedShapes[] = {
    {SSD_BF16, 64, 128, 256}, {SSD_BF16, 64, 128, 128}, {SSD_BF16, 64, 128, 64},
    {SSD_BF16, 16, 16, 64},   {SSD_F32, 16, 16, 64},    {SSD_F32, 64, 128, 64},
    {SSD_BF16, 16, 16, 256},  {SSD_F32, 16, 16, 256},   {SSD_F32, 64, 128, 256},
    {SSD_BF16, 16, 128, 64},  {SSD_BF16, 16, 128, 256}, {SSD_BF16, 64, 16, 64},
    {SSD_BF16, 64, 16, 256},  {SSD_F32, 16, 128, 64},   {SSD_F32, 16, 128, 256},
    {SSD_F32, 64, 16, 64},    {SSD_F32, 64, 16, 256},
};
const int kNumChunkedShapes = sizeof(kChunkedShapes) / sizeof(kChunkedShapes[0]);

bool decode_supports_n(int N) {
  return N == 16 || N == 32 || N == 64 || N == 128 || N == 256;
}

static bool valid_dtype(int32_t d) { return d == SSD_F32 || d == SSD_BF16; }
static bool valid_state_dtype(int32_t d) { return valid_dtype(d) || d == SSD_F16; }

ssd_status plan_prefill(const ssd_prefill_args* a, PrefillPlan* plan) {
  if (!a || !plan) return SSD_ERR_NULL_POINTER;
  *plan = PrefillPlan{};
  if (a->T < 0 || a->num_seqs < 0 || a->num_chunks < 0) return SSD_ERR_BAD_SHAPE;
  if (a->H < 1 || a->P < 1 || a->G < 1 || a->N < 1 || a->chunk_size < 1)
    return SSD_ERR_BAD_SHAPE;
  if (a->H % a->G != 0) return SSD_ERR_BAD_SHAPE;
  if (!valid_dtype(a->in_dtype)) return SSD_ERR_BAD_SHAPE;
  if (a->a_kind != SSD_A_SCALAR && a->a_kind != SSD_A_DIAG) return SSD_ERR_BAD_SHAPE;
  if (a->num_seqs == 0) {
    // an empty batch: nothing to do
    if (a->T != 0 || a->num_chunks != 0) return SSD_ERR_BAD_SHAPE;
    return SSD_OK;
  }
  // every sequence has >= 1 token and every chunk >= 1 token
  if (a->T < a->num_seqs || a->num_chunks < a->num_seqs || a->num_chunks > a->T)
    return SSD_ERR_BAD_SHAPE;
  const int64_t HP = int64_t(a->H) * a->P;
  const int64_t state = HP * a->N;
  if (a->x_stride_t < HP || a->y_stride_t < HP || a->dt_stride_t < a->H ||
      a->bc_stride_t < int64_t(a->G) * a->N)
    return SSD_ERR_BAD_SHAPE;
  if (!a->x || !a->dt || !a->B || !a->C || !a->y || !a->A) return SSD_ERR_NULL_POINTER;
  if (!a->cu_seqlens || !a->cu_chunk_seqlens || !a->seq_idx || !a->last_chunk_indices)
    return SSD_ERR_NULL_POINTER;
  const bool need_pool = a->has_initial_state != nullptr || a->write_final_to_pool != 0;
  if (need_pool) {
    if (!a->state_pool || !a->state_indices) return SSD_ERR_NULL_POINTER;
  }
  if (a->state_pool) {
    if (a->num_slots < 1 || a->slot_stride < state) return SSD_ERR_BAD_SHAPE;
  }
  if (std::isnan(a->dt_min) || std::isnan(a->dt_max) || a->dt_min > a->dt_max)
    return SSD_ERR_BAD_SHAPE;
  if (!valid_state_dtype(a->state_dtype)) return SSD_ERR_BAD_SHAPE;
  // the all cache mode: one pool entry per cache block of block_size tokens
  if (a->block_size < 0) return SSD_ERR_BAD_SHAPE;
  if (a->block_size > 0) {
    if (a->block_size % a->chunk_size != 0 || a->idx_stride < 1) return SSD_ERR_BAD_SHAPE;
    if (!a->state_pool || !a->state_indices || !a->num_computed) return SSD_ERR_NULL_POINTER;
    if (a->has_initial_state && !a->block_idx_last_computed) return SSD_ERR_NULL_POINTER;
    if (a->write_final_to_pool && !a->block_idx_last_scheduled) return SSD_ERR_NULL_POINTER;
  }

  const int64_t C = a->num_chunks;
  if (a->a_kind == SSD_A_DIAG) {
    if (a->P != 1 || a->G != 1) return SSD_ERR_BAD_SHAPE;
    if (a->N != kDiagN) return SSD_ERR_UNSUPPORTED;
    if (a->dA_cumsum_out || a->cb_out || a->chunk_local_states_out) return SSD_ERR_UNSUPPORTED;
    plan->kind = PrefillKind::kDiag;
    plan->ws_bytes = 0;
    return SSD_OK;
  }

  if (a->P == 1) {
    // head_dim 1: the sequential scan with A[h] on every state (the MFMA form would contract
    // over one column); any chunk size, the per-step debug outputs are not produced
    if (!scalar_p1_supports_n(a->N)) return SSD_ERR_UNSUPPORTED;
    if (a->dA_cumsum_out || a->cb_out || a->chunk_local_states_out) return SSD_ERR_UNSUPPORTED;
    plan->kind = PrefillKind::kDiag;
    plan->ws_bytes = 0;
    return SSD_OK;
  }

  int variant = -1;
  for (int i = 0; i < kNumChunkedShapes; ++i) {
    const ChunkedShape& s = kChunkedShapes[i];
    if (s.dtype == a->in_dtype && s.P == a->P && s.N == a->N && s.CS == a->chunk_size) {
      variant = i;
      break;
    }
  }
  if (variant < 0) return SSD_ERR_UNSUPPORTED;
  // The chunked kernels factor exp(c_l - c_s) through reference points inside a chunk,
  // which needs delta >= 0 (a monotone cumsum of delta*A): dt_min must not be negative.
  if (!(a->dt_min >= 0.f)) return SSD_ERR_UNSUPPORTED;
  plan->kind = PrefillKind::kChunked;
  plan->variant = variant;

  size_t off = 0;
  const size_t esz = a->in_dtype == SSD_BF16 ? 2 : 4;
  const size_t cs = size_t(a->chunk_size);
  plan->off_cb = off;
  off = align_up(off + size_t(C) * a->G * size_t(cb_frag_base(int(cs / 16))) * 512 * esz, 256);
  plan->off_bt = off;
  off = align_up(off + size_t(C) * a->G * a->N * cs * esz, 256);
  plan->chain = chain_supported(a->in_dtype, a->P, a->N, a->chunk_size);
  plan->off_dc = off;   // the chain kernel forms delta and the cumsum itself
  if (!plan->chain) off = align_up(off + size_t(C) * a->H * 2 * cs * sizeof(float), 256);
  plan->off_cf = off;
  off = align_up(off + size_t(C) * a->G * cs * size_t(a->N < 32 ? 32 : a->N) * esz, 256);
  plan->off_ord = off;
  off = align_up(off + size_t(a->num_seqs) * sizeof(int32_t), 256);
  if (plan->chain) {
    plan->off_flag = off;
    off = align_up(off + size_t(C) * a->H * kChainWaves * sizeof(int32_t), 256);
    // the work-item table: C * H items, each XCD's run at most total / 8 + one chain of
    // at most C - S + 1 chunks (rounding: + 1), padded to 8 per row
    if (chain_ordered(a->num_seqs, C, a->H)) {
      plan->chain_grid = int(C * a->H + kXcds * (C - a->num_seqs + 2));
      plan->off_items = off;
      off = align_up(off + size_t(plan->chain_grid) * sizeof(int32_t), 256);
    } else {
      plan->chain_grid = int(C * kXcds * ((a->H + kXcds - 1) / kXcds));
      plan->off_items = 0;
    }
    plan->off_ring = off;
    if (!a->chunk_states_out)
      off = align_up(off + size_t(a->num_seqs) * a->H * 2 * size_t(state / a->H) * sizeof(float), 256);
  }
  plan->off_blk = off;
  if (a->block_size > 0) off = align_up(off + size_t(C) * sizeof(int32_t), 256);
  plan->ws_bytes = off;
  return SSD_OK;
}

ssd_status check_decode(const ssd_decode_args* a) {
  if (!a) return SSD_ERR_NULL_POINTER;
  if (a->B_pad < 0) return SSD_ERR_BAD_SHAPE;
  if (a->ntok < 1 || a->H < 1 || a->P < 1 || a->G < 1 || a->N < 1) return SSD_ERR_BAD_SHAPE;
  if (a->H % a->G != 0) return SSD_ERR_BAD_SHAPE;
  if (!valid_dtype(a->in_dtype)) return SSD_ERR_BAD_SHAPE;
  if (a->a_kind != SSD_A_SCALAR && a->a_kind != SSD_A_DIAG) return SSD_ERR_BAD_SHAPE;
  if (!valid_state_dtype(a->state_dtype)) return SSD_ERR_BAD_SHAPE;
  if (a->ntok > kDecodeMaxTokens) return SSD_ERR_UNSUPPORTED;
  if (a->a_kind == SSD_A_DIAG) {
    // Mamba1: one channel per head position, one B/C group, dstate 16
    if (a->P != 1 || a->G != 1) return SSD_ERR_BAD_SHAPE;
    if (a->N != kDiagN) return SSD_ERR_UNSUPPORTED;
  } else if (!decode_supports_n(a->N) || int64_t(a->P) * a->N > kDecodeMaxStateElems) {
    return SSD_ERR_UNSUPPORTED;
  }
  if (std::isnan(a->dt_min) || std::isnan(a->dt_max) || a->dt_min > a->dt_max)
    return SSD_ERR_BAD_SHAPE;
  // the all cache mode: one token per row, no speculative restore
  if (a->idx_stride < 0) return SSD_ERR_BAD_SHAPE;
  if (a->idx_stride > 0 && (a->ntok != 1 || a->num_accepted_tokens)) return SSD_ERR_BAD_SHAPE;
  if (a->B_pad == 0) return SSD_OK;
  if (!a->x || !a->dt || !a->B || !a->C || !a->y || !a->A || !a->state_pool ||
      !a->state_indices)
    return SSD_ERR_NULL_POINTER;
  if (a->idx_stride > 0 && (!a->block_idx_last_computed || !a->block_idx_last_scheduled))
    return SSD_ERR_NULL_POINTER;
  if (a->num_slots < 1 || a->slot_stride < int64_t(a->H) * a->P * a->N)
    return SSD_ERR_BAD_SHAPE;
  return SSD_OK;
}

}  // namespace ssd

// ----------------------------------------------------------------------------------------
// C ABI: library information and the chunk-metadata builder
// ----------------------------------------------------------------------------------------
extern "C" {

int ssd_abi_version(void) { return SSD_ABI_VERSION; }

const char* ssd_status_string(ssd_status s) {
  switch (s) {
    case SSD_OK: return "ok";
    case SSD_ERR_NULL_POINTER: return "a required pointer is NULL";
    case SSD_ERR_BAD_SHAPE: return "a size or stride is out of range or inconsistent";
    case SSD_ERR_BAD_METADATA: return "inconsistent sequence metadata";
    case SSD_ERR_UNSUPPORTED: return "shape or dtype not instantiated";
    case SSD_ERR_CAPACITY: return "output capacity too small";
    case SSD_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case SSD_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

// Walks the sequences once; when `emit` is false only counts.  The first chunk of a
// resumed sequence closes the open chunk (cs - nc % cs tokens at most); after it every
// chunk holds min(cs, remaining) tokens.
static ssd_status chunk_walk(int32_t S, const int32_t* cu, const int32_t* nc, int32_t cs,
                             int32_t capacity, bool emit, int32_t* cu_chunk,
                             int32_t* seq_idx, int32_t* last, int32_t* count_out) {
  if (!count_out || (S > 0 && !cu)) return SSD_ERR_NULL_POINTER;
  if (S < 0 || cs <= 0) return SSD_ERR_BAD_SHAPE;
  if (cu && cu[0] != 0) return SSD_ERR_BAD_METADATA;
  int64_t count = 0;
  for (int32_t r = 0; r < S; ++r) {
    const int64_t new_tokens = int64_t(cu[r + 1]) - cu[r];
    const int64_t done = nc ? nc[r] : 0;
    if (new_tokens < 1 || done < 0) return SSD_ERR_BAD_METADATA;
    // a sequence's absolute positions (num_computed + new tokens) must fit in int32: the
    // kernels place block and chunk ends with 32-bit positions
    if (done + new_tokens > std::numeric_limits<int32_t>::max()) return SSD_ERR_BAD_METADATA;
    int64_t left = new_tokens;
    if (done % cs != 0) {
      const int64_t open = cs - done % cs;
      left -= (open < left ? open : left);
      ++count;
    }
    count += (left + cs - 1) / cs;
    if (count > std::numeric_limits<int32_t>::max()) return SSD_ERR_BAD_METADATA;
  }
  *count_out = int32_t(count);
  if (!emit) return SSD_OK;
  if (!cu_chunk || !seq_idx || (S > 0 && !last)) return SSD_ERR_NULL_POINTER;
  if (count > capacity) return SSD_ERR_CAPACITY;

  int32_t k = 0;
  cu_chunk[0] = 0;
  for (int32_t r = 0; r < S; ++r) {
    int64_t pos = cu[r];
    const int64_t end = cu[r + 1];
    const int64_t done = nc ? nc[r] : 0;
    if (done % cs != 0) {
      const int64_t open = cs - done % cs;
      pos += (open < end - pos ? open : end - pos);
      cu_chunk[k + 1] = int32_t(pos);
      seq_idx[k] = r;
      ++k;
    }
    while (pos < end) {
      pos += (cs < end - pos ? cs : end - pos);
      cu_chunk[k + 1] = int32_t(pos);
      seq_idx[k] = r;
      ++k;
    }
    last[r] = k - 1;
  }
  return SSD_OK;
}

ssd_status ssd_chunk_metadata_count(int32_t num_seqs, const int32_t* cu_seqlens,
                                    const int32_t* num_computed, int32_t chunk_size,
                                    int32_t* num_chunks_out) {
  return chunk_walk(num_seqs, cu_seqlens, num_computed, chunk_size, 0, false, nullptr,
                    nullptr, nullptr, num_chunks_out);
}

ssd_status ssd_build_chunk_metadata(int32_t num_seqs, const int32_t* cu_seqlens,
                                    const int32_t* num_computed, int32_t chunk_size,
                                    int32_t capacity, int32_t* cu_chunk_seqlens,
                                    int32_t* seq_idx, int32_t* last_chunk_indices,
                                    int32_t* num_chunks_out) {
  return chunk_walk(num_seqs, cu_seqlens, num_computed, chunk_size, capacity, true,
                    cu_chunk_seqlens, seq_idx, last_chunk_indices, num_chunks_out);
}

}  // extern "C"
