// ssd_debug.hip -- the SSD_DEBUG checks of the distinct-slot precondition.
//
// The prefill and the decode update the state pool in place, so a pool entry that two
// sequences (or two decode rows) both touch is a race.  Distinct entries are a documented
// precondition of both calls; when the environment variable SSD_DEBUG is set (to anything
// but "0") each call first launches one of the kernels below on its stream, which raises
// SSD_DEVERR_DUPLICATE_SLOT in *device_error_flag when two different sequences or rows
// touch the same slot.  The check is O(n^2) in the entries touched: a debugging aid, not a
// production path.  Entries that are out of range, and padding rows, are left to the
// call's own kernels.
#include <cstdlib>
#include <cstring>

#include "ssd_params.h"

namespace ssd {
namespace {

// Entry col of decode row r if the row touches it (read or written), else -1.  Normal mode:
// every column of a live row (the source is one of them); all cache mode: the
// last-computed (source) and last-scheduled (destination) columns of a live row.
__device__ int decode_touched(const DecodeParams& p, int r, int col) {
  if (p.idx_stride > 0) {
    const int ls = p.blk_last_sched[r], lc = p.blk_last_comp[r];
    if (ls < 0 || ls >= p.idx_stride || lc < 0 || lc >= p.idx_stride) return -1;
    const int64_t row = int64_t(r) * p.idx_stride;
    if (p.idx[row + ls] == p.null_id) return -1;
    if (col != ls && col != lc) return -1;
    const int s = p.idx[row + col];
    return s >= 0 && s < p.num_slots ? s : -1;
  }
  const int64_t row = int64_t(r) * p.ntok;
  if (col >= p.ntok || p.idx[row] == p.null_id) return -1;
  const int s = p.idx[row + col];
  return s >= 0 && s < p.num_slots ? s : -1;
}

__global__ __launch_bounds__(256) void k_check_decode_slots(DecodeParams p, int width) {
  const int64_t n = int64_t(p.B_pad) * width;
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const int r = int(i / width), s = decode_touched(p, r, int(i % width));
  if (s < 0) return;
  for (int64_t k = 0; k < n; ++k) {
    const int rk = int(k / width);
    if (rk != r && decode_touched(p, rk, int(k % width)) == s) {
      raise_flag(p.flag, SSD_DEVERR_DUPLICATE_SLOT);
      return;
    }
  }
}

// Entry col of sequence r if the prefill reads or writes it, else -1.  Normal mode: the
// sequence's slot (column 0) when it reads an initial state or writes the final one; all
// cache mode: the columns from the initial state's (or the first block end's) to the last
// block end's or, with write_final, the last-scheduled one.
__device__ int prefill_touched(const PrefillParams& p, int r, int col) {
  const bool init = p.has_init && p.has_init[r];
  int lo = 0, hi = -1;
  if (p.block_size > 0) {
    const int64_t nc = p.num_computed[r], L = int64_t(p.cu_seqlens[r + 1]) - p.cu_seqlens[r];
    if (nc < 0 || L < 1) return -1;
    lo = int(nc / p.block_size);
    if (init) lo = min(lo, p.blk_last_comp[r]);
    hi = p.write_final ? p.blk_last_sched[r] : int((nc + L) / p.block_size) - 1;
  } else if (init || p.write_final) {
    hi = 0;
  }
  if (col < max(lo, 0) || col > hi || col >= p.idx_stride) return -1;
  const int s = p.state_idx[int64_t(r) * p.idx_stride + col];
  return s >= 0 && s < p.num_slots ? s : -1;
}

__global__ __launch_bounds__(256) void k_check_prefill_slots(PrefillParams p) {
  const int64_t n = int64_t(p.S) * p.idx_stride;
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const int r = int(i / p.idx_stride), s = prefill_touched(p, r, int(i % p.idx_stride));
  if (s < 0) return;
  for (int64_t k = 0; k < n; ++k) {
    const int rk = int(k / p.idx_stride);
    if (rk != r && prefill_touched(p, rk, int(k % p.idx_stride)) == s) {
      raise_flag(p.flag, SSD_DEVERR_DUPLICATE_SLOT);
      return;
    }
  }
}

}  // namespace

bool debug_checks_enabled() {
  const char* v = std::getenv("SSD_DEBUG");
  return v && *v && std::strcmp(v, "0") != 0;
}

hipError_t launch_decode_slot_check(const DecodeParams& p, hipStream_t s) {
  if (!p.flag || !p.idx || p.B_pad <= 0) return hipSuccess;
  const int width = p.idx_stride > 0 ? p.idx_stride : p.ntok;
  const int64_t n = int64_t(p.B_pad) * width;
  hipLaunchKernelGGL(k_check_decode_slots, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, p,
                     width);
  return hipGetLastError();
}

hipError_t launch_prefill_slot_check(const PrefillParams& p, hipStream_t s) {
  if (!p.flag || !p.pool || !p.state_idx || p.S <= 0) return hipSuccess;
  const int64_t n = int64_t(p.S) * p.idx_stride;
  hipLaunchKernelGGL(k_check_prefill_slots, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ssd
