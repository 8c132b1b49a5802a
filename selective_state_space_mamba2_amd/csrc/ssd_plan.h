// ssd_plan.h -- host-side planning shared by the C-ABI entry points and the launchers.
// Plain C++ (no HIP headers): validation, instantiation lookup and workspace layout.
#pragma once

#include <cstddef>
#include <cstdint>

#include "ssd.h"

namespace ssd {

// Which prefill implementation runs.
// kDiag: the sequential scan of a one-element head (SSD_A_DIAG, or SSD_A_SCALAR with P == 1).
enum class PrefillKind { kNone = 0, kChunked = 1, kDiag = 2 };

// Workspace carve-up of one prefill call (byte offsets into the caller's workspace).
struct PrefillPlan {
  PrefillKind kind = PrefillKind::kNone;
  int variant = -1;          // index into the chunked-kernel instantiation table
  size_t ws_bytes = 0;
  size_t off_cb = 0;         // input dtype, per (chunk, group): the C.B^T blocks of every
                             // row tile, cb_frag_base(cs/16) fragments of 512 values
  size_t off_bt = 0;         // input dtype [C, G, N * cs]: B^T per chunk and group
  size_t off_dc = 0;         // fp32 [C, H, 2, cs]: cumsum of delta*A, then delta (march
                             // kernels only)
  size_t off_cf = 0;         // input dtype [C, G, cs * max(N, 32)]: C rows as fragments
  size_t off_ord = 0;        // int32 [S]: sequence dispatch order of the march kernel
  bool chain = false;        // the chunk-chain kernel runs (else a march kernel)
  size_t off_flag = 0;       // int32 [C, H, kChainWaves]: chain publication flags
  size_t off_items = 0;      // int32 [chain_grid]: the chain kernel's work items (0 bytes
                             // when the batch is too large to order)
  int chain_grid = 0;        // workgroups of the chain kernel
  size_t off_ring = 0;       // fp32 [S, H, 2, P, N]: published states when no chunk-state
                             // output is given (0 bytes otherwise)
  size_t off_blk = 0;        // int32 [C]: the all cache mode's pool slot for every chunk's
                             // end state, -1 for none (0 bytes when the mode is off)
};

// Wavefronts per chunk-chain workgroup; each publishes its share of the state under a
// flag of its own, so there are kChainWaves flags per (chunk, head).
constexpr int kChainWaves = 4;
// The prep kernel orders the chain's work items (one workgroup, with every sequence and
// chunk in LDS, so the batch is bounded); larger batches run the chunks in index order.
constexpr int kChainOrderMaxSeqs = 1024;
constexpr int kChainOrderMaxChunks = 6144;
constexpr bool chain_ordered(int64_t S, int64_t C, int64_t H) {
  return S <= kChainOrderMaxSeqs && C <= kChainOrderMaxChunks && C * H <= (int64_t(1) << 22);
}
// Shapes that run the chunk-chain kernel (bf16, head dim 64, dstate and chunk size
// multiples of 128, at most one token per thread of the workgroup); the others run the
// march kernel.
constexpr bool chain_supported(int dtype, int P, int N, int CS) {
  return dtype == SSD_BF16 && P == 64 && N % 128 == 0 && CS % 128 == 0 && CS <= 64 * kChainWaves;
}

// C.B^T fragments of the 16-row tiles 0..i-1 of a chunk: tile i needs the 32-token blocks
// 0..i/2 (one fragment each).
constexpr int cb_frag_base(int i) { return (i / 2) * (i / 2 + 1) + (i % 2) * (i / 2 + 1); }

// Placement of the march kernel's work items on the 8 XCDs of the device.  Items (one per
// sequence, head and head-dim slice, in sequence dispatch order) are cut into nblocks =
// 8 * ceil(S*G / 8) contiguous blocks of bsize items; block j runs on the XCD that
// receives the workgroup ids w with w % 8 == j % 8 (one XCD per residue: the round-robin
// dispatch starts at an XCD that varies between launches).  The workgroups that read the same
// chunk's C.B^T / B^T / C fragments (one sequence and group) thus share an L2.  The grid
// has nblocks * bsize workgroups; ids past the last item exit at once.
struct MarchGrid {
  int items, nblocks, bsize;
};
constexpr int kXcds = 8;
constexpr MarchGrid march_grid(int S, int G, int H, int ps) {
  const int items = S * H * ps;
  const int nblocks = kXcds * ((S * G + kXcds - 1) / kXcds);
  return MarchGrid{items, nblocks, (items + nblocks - 1) / nblocks};
}

// One instantiated chunked-prefill shape.
struct ChunkedShape {
  int dtype;   // ssd_dtype
  int P, N, CS;
};

// The table of chunked instantiations (defined next to the kernels' dispatch table, but
// the shapes are plain data so the host can validate without a device).
extern const ChunkedShape kChunkedShapes[];
extern const int kNumChunkedShapes;

// Decode: supported dstates (template instantiations of the update kernel) and limits.
constexpr int kDecodeMaxTokens = 16;
constexpr int kDecodeMaxStateElems = 16384;   // P * N per head
bool decode_supports_n(int N);

// Diagonal (Mamba1) scan: the one instantiated dstate.  The same sequential scan runs
// the scalar-A recurrence at head_dim 1 with these dstates:
constexpr int kDiagN = 16;
constexpr bool scalar_p1_supports_n(int N) { return N == 16 || N == 128; }

ssd_status plan_prefill(const ssd_prefill_args* a, PrefillPlan* plan);
ssd_status check_decode(const ssd_decode_args* a);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace ssd
