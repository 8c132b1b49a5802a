// ssd_diag.hip -- sequential selective scan with a one-element head: Mamba1's per-(channel,
// state) diagonal A, and Mamba2's scalar A per head at head_dim 1.
//
// The S6 model of "[vLLM] Mamba (SSM)" (paper key content) with A[channel, state]:
//   h[c,n] = exp(delta[t,c] A[c,n]) h[c,n] + delta[t,c] x[t,c] B[t,n];  y[t,c] = sum_n C[t,n] h[c,n] + D[c] x[t,c]
// Mamba1 has no chunk notion of its own, so the chunk size only sets where state
// checkpoints are written ("vLLM Mamba2 SSD kernel warm-up", config/model.py section).
// The Mamba2 recurrence with head_dim 1 is the same scan with A[c, n] = A[c] for every n
// (one decay per (token, head), so one exponential instead of N) and B/C taken from the
// head's group g = c / (H / G): its MFMA form would contract over a single column.
//
// This path is bound by the exponential and VALU work, not by a contraction, so it runs on
// the vector ALUs: one workgroup owns CH channels of one group of one sequence and walks
// its tokens in order; each channel's N states are spread over LPC adjacent lanes (SPL
// states each) and y is an LPC-lane reduction.  Token tiles of delta, x, B and C are staged
// through LDS with coalesced loads (64 channels = 128 B per token for bf16), delta is
// prepared once per (token, channel) while staging, and y leaves through an LDS tile as
// coalesced rows.  Checkpoints are written at the chunk ends listed by the chunk metadata.
//
// Two grids: k_diag_scan, one workgroup per (sequence, group, block of CH channels), and
// for Mamba1 (N = 16, one group) k_diag_scan_mixed, which covers part of the channels with
// 32-channel workgroups of two states per lane when that spreads the work more evenly over
// the SIMDs (the host picks it with a model of the dispatch, see mamba1_grid).
#include <algorithm>
#include <atomic>
#include <cstdint>
#include <type_traits>

#include "ssd_params.h"

namespace ssd {

#ifndef SSD_DIAG_UNROLL
#define SSD_DIAG_UNROLL 4
#endif
#ifndef SSD_DIAG_SPL
#define SSD_DIAG_SPL 4
#endif

// NS states per channel, SPL per lane: a channel's states sit on LPC = NS/SPL adjacent
// lanes and a workgroup owns CH = 256 / LPC channels.
template <int NS, int SPL>
struct DiagCfg {
  static_assert((SPL % 4 == 0 || SPL == 2) && NS % SPL == 0, "states move 4 (or 2) at a time");
  static constexpr int N = NS, LPC = N / SPL, CH = 256 / LPC;
};

constexpr int kDiagTT = 32;   // tokens per LDS tile

// A workgroup's LDS: one token tile of delta, x and y per channel and of B and C per state.
// Declared by the kernels (one object shared by every body a kernel inlines).
template <int NS, int SPL>
struct DiagSmem {
  static constexpr int CH = DiagCfg<NS, SPL>::CH;
  __attribute__((aligned(16))) float d[kDiagTT][CH];
  __attribute__((aligned(16))) float x[kDiagTT][CH];
  __attribute__((aligned(16))) float y[kDiagTT][CH];
  __attribute__((aligned(16))) float b[kDiagTT][NS];
  __attribute__((aligned(16))) float c[kDiagTT][NS];
};

// The 16-byte path of x, delta and y (bf16, 8 channels per thread): whole 8-channel groups
// (H/G % 8 == 0), row strides in whole 8-element units and 16-byte aligned tensors.
template <typename T, int CH>
__device__ __forceinline__ bool diag_vec_ok(const PrefillParams& p) {
  constexpr bool kVecT = std::is_same<T, bf16_t>::value && CH % 8 == 0 && 256 / (CH / 8) >= kDiagTT;
  return kVecT && (p.H / p.G) % 8 == 0 && p.x_st % 8 == 0 && p.dt_st % 8 == 0 && p.y_st % 8 == 0 &&
         ((reinterpret_cast<uintptr_t>(p.x) | reinterpret_cast<uintptr_t>(p.dt) |
           reinterpret_cast<uintptr_t>(p.y)) & 15) == 0;
}

// The SPL states of a lane to and from the pool (any pool dtype) and the fp32 checkpoint
// output: four at a time, or two (8 bytes of fp32, 4 of a 2-byte pool) when SPL is 2.
template <int SPL>
__device__ __forceinline__ void diag_pool_ld(const void* pool, int kind, int64_t e, float* h) {
  if constexpr (SPL == 2) {
    if (kind == SSD_F32) {
      const float2_v v = *reinterpret_cast<const float2_v*>(static_cast<const float*>(pool) + e);
      h[0] = v.x; h[1] = v.y;
    } else {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(pool) + e);
      h[0] = kind == SSD_BF16 ? bf16_to_f32(bf16_t(w & 0xffffu)) : f16_to_f32(w);
      h[1] = kind == SSD_BF16 ? bf16_to_f32(bf16_t(w >> 16)) : f16_to_f32(w >> 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < SPL; i += 4) {
      const float4_v v = pool_ld4(pool, kind, e + i);
      h[i] = v.x; h[i + 1] = v.y; h[i + 2] = v.z; h[i + 3] = v.w;
    }
  }
}
template <int SPL>
__device__ __forceinline__ void diag_pool_st(void* pool, int kind, int64_t e, const float* h) {
  if constexpr (SPL == 2) {
    if (kind == SSD_F32) {
      *reinterpret_cast<float2_v*>(static_cast<float*>(pool) + e) = float2_v{h[0], h[1]};
    } else {
      *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(pool) + e) =
          kind == SSD_BF16 ? pack_bf16x2(h[0], h[1]) : pack_f16x2(h[0], h[1]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < SPL; i += 4)
      pool_st4(pool, kind, e + i, float4_v{h[i], h[i + 1], h[i + 2], h[i + 3]});
  }
}

// Sum of v over the aligned group of LPC (2, 4, 8 or 16) lanes, on every lane of the
// group: DPP quad permutations (lane ^ 1, then lane ^ 2), then rotations by 4 and 8 lanes
// inside the 16-lane row, feed the adds directly, with no LDS trip.
template <int LPC>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(LPC == 1 || LPC == 2 || LPC == 4 || LPC == 8 || LPC == 16,
                "lanes per channel within a row");
  if constexpr (LPC >= 2)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  if constexpr (LPC >= 4)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  if constexpr (LPC == 8) {
    // the other quad of the 8-lane half row: row_half_mirror (lane i of the half reads 7-i)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
  }
  if constexpr (LPC >= 16) {
    // quad sums q0..q3 of the row: + row_ror:4 gives q_i + q_(i+1), + row_ror:8 the total
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, true));
  }
  return v;
}

// Workgroups of one sequence: G groups x ceil(H/G / CH) channel blocks, so the channels of
// a workgroup share one B/C group.
__host__ __device__ __forceinline__ int diag_blocks_per_group(int H, int G, int CH) {
  return (H / G + CH - 1) / CH;
}

// kScalarA: A is [H] (Mamba2 at head_dim 1), else [H, NS] (Mamba1).
// The channels of one workgroup: [c0, c0 + nch) of group g, sequence r; `lead` is the
// workgroup that reports the sequence's metadata and slot faults (one per sequence).
struct DiagWork {
  int r, g, c0, nch;
  bool lead;
};

// kVec: the 16-byte path (diag_vec_ok holds), a template argument so that the two paths'
// loads never meet in one loop (a load of one path would otherwise be waited for in the
// other).
template <typename T, int NS, int SPL, bool kScalarA, bool kVec>
__device__ __forceinline__ void diag_body(const PrefillParams& p, const DiagWork w,
                                          DiagSmem<NS, SPL>& sm) {
  using Cfg = DiagCfg<NS, SPL>;
  constexpr int N = NS;                // states per channel
  constexpr int LPC = Cfg::LPC;        // lanes per channel
  constexpr int CH = Cfg::CH;          // channels per workgroup
  constexpr int TT = kDiagTT;          // tokens per LDS tile
  constexpr int U = SSD_DIAG_UNROLL;   // tokens per step of the scan (divides TT)
  constexpr int NA = kScalarA ? 1 : SPL;   // decay factors per lane and token
  static_assert(TT % U == 0, "unroll");
  auto& s_d = sm.d;
  auto& s_x = sm.x;
  auto& s_y = sm.y;
  auto& s_b = sm.b;
  auto& s_c = sm.c;

  const int tid = threadIdx.x;
  const int r = w.r, g = w.g, c0 = w.c0, nch = w.nch;
  const int H = p.H, HPG = p.H / p.G;
  const int cl = tid / LPC, ng = tid % LPC;
  const int c = c0 + cl;
  const bool valid = cl < nch;

  const int t0 = p.cu_seqlens[r], t1 = p.cu_seqlens[r + 1];
  int k = r == 0 ? 0 : p.last_chunk[r - 1] + 1;
  const int klast = p.last_chunk[r];
  const bool first_wg = w.lead;
  if (t0 < 0 || t1 > p.T || t1 <= t0 || k < 0 || klast < k || klast >= p.C || p.cu_chunk[k] != t0 ||
      p.cu_chunk[klast + 1] != t1) {
    if (tid == 0 && first_wg) raise_flag(p.flag, SSD_DEVERR_CHUNK_RANGE);
    return;
  }
  int next_end = p.cu_chunk[k + 1];

  float A2[NA];
  float h[SPL];
#pragma unroll
  for (int i = 0; i < SPL; ++i) h[i] = 0.f;
  // pool entries: the initial state (read only with has_initial_state) and the final
  // state (written only with write_final); in the all cache mode the block_idx_last_computed
  // and block_idx_last_scheduled entries, plus one entry per block end below
  const bool report = tid == 0 && first_wg;
  const SeqSlots ss = seq_slots(p, r, true, true, report);
  const int src = (ss.src >= 0 && p.has_init && p.has_init[r]) ? ss.src : -1;
  const int fin = p.write_final ? ss.fin : -1;
  if (valid) {
#pragma unroll
    for (int i = 0; i < NA; ++i) A2[i] = (kScalarA ? p.A[c] : p.A[c * N + ng * SPL + i]) * kLog2e;
    if (src >= 0) {
      diag_pool_ld<SPL>(p.pool, p.pool_kind, int64_t(src) * p.slot_stride + int64_t(c) * N + ng * SPL, h);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NA; ++i) A2[i] = 0.f;
  }
  const float Dc = (valid && p.D) ? p.D[c] : 0.f;

  const T* xg = static_cast<const T*>(p.x);
  const T* dg = static_cast<const T*>(p.dt);
  const T* bg = static_cast<const T*>(p.B) + int64_t(g) * N;
  const T* cg = static_cast<const T*>(p.Cm) + int64_t(g) * N;
  T* yg = static_cast<T*>(p.y);

  // A tile's inputs are fetched into registers one tile ahead (raw values; positions past
  // the sequence end read as zero) and written to LDS at the top of the tile's turn.
  constexpr int NE = TT * CH / 256;              // delta / x elements per thread
  constexpr int NBC = TT * 2 * (N / 4);          // B / C float4 items per tile
  constexpr int NBCI = (NBC + 255) / 256;        // ... per thread
  T rd[NE], rx[NE];
  T rbc[NBCI][4];   // raw: converted when staged, so the fetch does not wait for its loads
  // Vector path (bf16, 8 channels per thread): thread t owns channels 8*(t % VPR) .. +7 of
  // tile row t / VPR (VPR = CH / 8 threads per row; rows past the tile idle), moved as one
  // 16-byte access per tensor.  Otherwise one element per access.
  constexpr int VPR = CH / 8;
  constexpr bool vec = kVec;
  const int vtt = tid / VPR, vc8 = (tid % VPR) * 8, vch = c0 + vc8;
  const bool vin = vc8 < nch;
  u32x4_v vd = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
  auto fetch = [&](int tb) {
    const int nt = min(TT, t1 - tb);
    // B / C first: their zero fill then never waits behind the x / delta loads
#pragma unroll
    for (int u = 0; u < NBCI; ++u) {
      const int e = u * 256 + tid;
#pragma unroll
      for (int i = 0; i < 4; ++i) rbc[u][i] = T(0);
      const int tt = e / (2 * (N / 4)), q = e % (2 * (N / 4));
      const int which = q / (N / 4), n4 = q % (N / 4);
      if (e < NBC && tt < nt) {
        const T* src = (which ? cg : bg) + int64_t(tb + tt) * p.bc_st + n4 * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) rbc[u][i] = src[i];
      }
    }
    if constexpr (vec) {
      const bool in = vtt < nt && vin;
      vd = in ? *reinterpret_cast<const u32x4_v*>(dg + int64_t(tb + vtt) * p.dt_st + vch)
              : u32x4_v{0u, 0u, 0u, 0u};
      vx = in ? *reinterpret_cast<const u32x4_v*>(xg + int64_t(tb + vtt) * p.x_st + vch)
              : u32x4_v{0u, 0u, 0u, 0u};
    } else {
#pragma unroll
      for (int u = 0; u < NE; ++u) {
        const int e = u * 256 + tid, tt = e / CH, cc = e % CH;
        const bool in = tt < nt && cc < nch;
        const int64_t t = in ? tb + tt : t0;
        const int chc = in ? c0 + cc : 0;
        rd[u] = in ? dg[t * p.dt_st + chc] : T(0);
        rx[u] = in ? xg[t * p.x_st + chc] : T(0);
      }
    }
  };
  // per-thread constants of the staging: the dt bias of each channel this thread stages
  // (the 8 of its vector, or the one of its column: 256 is a multiple of CH)
  static_assert(256 % CH == 0, "one staging column per thread");
  constexpr int NB = vec ? 8 : 1;
  float bias[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int cc = vec ? vc8 + i : tid % CH;
    bias[i] = cc < nch ? p.prep.bias_of(c0 + cc) : 0.f;
  }
  // Wait here for the loads above (pool state, A, D, bias): a load still outstanding when
  // the tile loop starts would be waited for inside it, behind each tile's prefetch.
  __builtin_amdgcn_s_waitcnt(0);
  fetch(t0);
  for (int tb = t0; tb < t1; tb += TT) {
    const int nt = min(TT, t1 - tb);
    if constexpr (vec) {
      const bool in = vtt < nt && vin;
      float dv8[8], xv8[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        xv8[2 * k] = __uint_as_float(vx[k] << 16);
        xv8[2 * k + 1] = __uint_as_float(vx[k] & 0xffff0000u);
        dv8[2 * k] = in ? p.prep.apply(__uint_as_float(vd[k] << 16), bias[2 * k]) : 0.f;
        dv8[2 * k + 1] = in ? p.prep.apply(__uint_as_float(vd[k] & 0xffff0000u), bias[2 * k + 1])
                            : 0.f;
      }
      if (vtt < TT) {
        *reinterpret_cast<float4_v*>(&s_d[vtt][vc8]) = float4_v{dv8[0], dv8[1], dv8[2], dv8[3]};
        *reinterpret_cast<float4_v*>(&s_d[vtt][vc8 + 4]) = float4_v{dv8[4], dv8[5], dv8[6], dv8[7]};
        *reinterpret_cast<float4_v*>(&s_x[vtt][vc8]) = float4_v{xv8[0], xv8[1], xv8[2], xv8[3]};
        *reinterpret_cast<float4_v*>(&s_x[vtt][vc8 + 4]) = float4_v{xv8[4], xv8[5], xv8[6], xv8[7]};
      }
    } else {
#pragma unroll
      for (int u = 0; u < NE; ++u) {
        const int e = u * 256 + tid, tt = e / CH, cc = e % CH;
        const bool in = tt < nt && cc < nch;
        s_d[tt][cc] = in ? p.prep.apply(to_f32(rd[u]), bias[0]) : 0.f;
        s_x[tt][cc] = to_f32(rx[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < NBCI; ++u) {
      const int e = u * 256 + tid;
      const int tt = e / (2 * (N / 4)), q = e % (2 * (N / 4));
      const int which = q / (N / 4), n4 = q % (N / 4);
      if (e < NBC)
        *reinterpret_cast<float4_v*>(which ? &s_c[tt][4 * n4] : &s_b[tt][4 * n4]) =
            float4_v{to_f32(rbc[u][0]), to_f32(rbc[u][1]), to_f32(rbc[u][2]), to_f32(rbc[u][3])};
    }
    __syncthreads();
    if (tb + TT < t1) fetch(tb + TT);


    // The tile is walked in segments that end at a checkpoint (a chunk end inside the tile)
    // or at the tile end.  Inside a segment tokens go U at a time with no branch, so the
    // exponentials and LDS reads of a group, which do not depend on h, are issued together
    // and only the state updates run in sequence.  Positions past nt hold delta = 0 (decay 1,
    // no input), which leaves h unchanged, so the last segment may round up to a multiple
    // of U.
    auto steps = [&](int tt, auto ucount) {
      constexpr int V = decltype(ucount)::value;
      float dv[V], xv[V], a[V][NA], bb[V][SPL], cc4[V][SPL];
#pragma unroll
      for (int u = 0; u < V; ++u) {
        dv[u] = s_d[tt + u][cl];
        xv[u] = s_x[tt + u][cl];
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
          bb[u][i] = s_b[tt + u][ng * SPL + i];
          cc4[u][i] = s_c[tt + u][ng * SPL + i];
        }
#pragma unroll
        for (int i = 0; i < NA; ++i) a[u][i] = __builtin_amdgcn_exp2f(dv[u] * A2[i]);
      }
      float acc[V];
#pragma unroll
      for (int u = 0; u < V; ++u) {
        const float dx = dv[u] * xv[u];
        acc[u] = 0.f;
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
          h[i] = a[u][kScalarA ? 0 : i] * h[i] + dx * bb[u][i];
          acc[u] += cc4[u][i] * h[i];
        }
      }
#pragma unroll
      for (int u = 0; u < V; ++u) {
        acc[u] = group_sum<LPC>(acc[u]) + Dc * xv[u];
        // y complete on every lane here: left to the branch below, the last add of each
        // sum moves into it and its permutation becomes a separate instruction
        asm volatile("" ::"v"(acc[u]));
      }
      if (ng == 0) {
#pragma unroll
        for (int u = 0; u < V; ++u) s_y[tt + u][cl] = acc[u];
      }
    };
    int tt = 0;
    while (tt < nt) {
      const int cut = next_end - tb;   // tokens of this tile up to the next checkpoint
      const bool ckpt = cut > tt && cut <= nt;
      if (ckpt) {
#pragma unroll 1
        for (; tt + U <= cut; tt += U) steps(tt, std::integral_constant<int, U>{});
#pragma unroll 1
        for (; tt < cut; ++tt) steps(tt, std::integral_constant<int, 1>{});
        if (valid && p.states) {   // end of chunk k: checkpoint
          diag_pool_st<SPL>(p.states, SSD_F32, (int64_t(k) * H + c) * N + ng * SPL, h);
        }
        if (valid && p.block_size > 0) {   // the all cache mode: a block ends here
          const int col = block_end_col(p, r, t0, p.cu_chunk[k], next_end, report);
          const int bslot = col >= 0 ? pool_slot(p, r, col, report) : -1;
          if (bslot >= 0) {
            diag_pool_st<SPL>(p.pool, p.pool_kind,
                              int64_t(bslot) * p.slot_stride + int64_t(c) * N + ng * SPL, h);
          }
        }
        ++k;
        next_end = k <= klast ? p.cu_chunk[k + 1] : -1;
      } else {
        // single tokens up to a multiple of U (after a checkpoint inside the tile), then
        // groups: an aligned group never reaches past the tile's TT rows
#pragma unroll 1
        for (; tt < nt && tt % U != 0; ++tt) steps(tt, std::integral_constant<int, 1>{});
#pragma unroll 1
        for (; tt < nt; tt += U) steps(tt, std::integral_constant<int, U>{});
      }
    }
    __syncthreads();
    if constexpr (vec) {
      if (vtt < nt && vin) {
        const float4_v a = *reinterpret_cast<const float4_v*>(&s_y[vtt][vc8]);
        const float4_v b = *reinterpret_cast<const float4_v*>(&s_y[vtt][vc8 + 4]);
        *reinterpret_cast<u32x4_v*>(yg + int64_t(tb + vtt) * p.y_st + vch) =
            u32x4_v{pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                    pack_bf16x2(b.z, b.w)};
      }
    } else {
      for (int e = tid; e < nt * CH; e += 256) {
        const int tt = e / CH, cc = e % CH;
        if (cc < nch) Elem<T>::store(yg + int64_t(tb + tt) * p.y_st + c0 + cc, s_y[tt][cc]);
      }
    }
    __syncthreads();
  }
  if (k != klast + 1 && tid == 0 && first_wg) raise_flag(p.flag, SSD_DEVERR_CHUNK_RANGE);
  if (valid && fin >= 0) {
    diag_pool_st<SPL>(p.pool, p.pool_kind, int64_t(fin) * p.slot_stride + int64_t(c) * N + ng * SPL, h);
  }
}

// One workgroup per (group, block of CH channels) and sequence (blockIdx.y).
template <typename T, int NS, int SPL, bool kScalarA>
__device__ __forceinline__ void diag_run(const PrefillParams& p, const DiagWork w,
                                         DiagSmem<NS, SPL>& sm) {
  if (diag_vec_ok<T, DiagCfg<NS, SPL>::CH>(p)) diag_body<T, NS, SPL, kScalarA, true>(p, w, sm);
  else diag_body<T, NS, SPL, kScalarA, false>(p, w, sm);
}

template <typename T, int NS, int SPL, bool kScalarA>
__global__ __launch_bounds__(256) void k_diag_scan(PrefillParams p) {
  __shared__ DiagSmem<NS, SPL> sm;
  constexpr int CH = DiagCfg<NS, SPL>::CH;
  const int HPG = p.H / p.G, nb = diag_blocks_per_group(p.H, p.G, CH);
  const int g = blockIdx.x / nb, jb = blockIdx.x % nb;
  diag_run<T, NS, SPL, kScalarA>(
      p, DiagWork{int(blockIdx.y), g, g * HPG + jb * CH, min(CH, HPG - jb * CH), blockIdx.x == 0},
      sm);
}

// Mamba1 (one group) in workgroups of two sizes: per sequence nbig blocks of 64 channels
// with 4 states per lane over channels [0, 64 nbig), then nsmall blocks of 32 channels with
// 2 states per lane over the rest; every sequence's large workgroups come first in the grid.
// Dispatched one workgroup per CU per pass, a grid of two large to one small workgroup puts
// two large and one small workgroup on every CU instead of three large ones on half of the
// CUs and two on the rest (the work of a small workgroup is about 0.6 of a large one's).
// The two small workgroups of one 64-channel block split each 128-byte row segment of x,
// delta and y; their workgroup ids differ by 8, which puts them on the same XCD (ids go
// round-robin over the 8 XCDs), so the segment is fetched into one L2, not two.
template <typename T>
__global__ __launch_bounds__(256) void k_diag_scan_mixed(PrefillParams p, int nbig, int nsmall) {
  __shared__ union {
    DiagSmem<kDiagN, 4> big;
    DiagSmem<kDiagN, 2> small;
  } sm;
  const int b = blockIdx.x;
  if (b < p.S * nbig) {
    const int r = b / nbig, j = b - r * nbig;
    diag_run<T, kDiagN, 4, false>(p, DiagWork{r, 0, 64 * j, 64, j == 0}, sm.big);
  } else {
    // ids base .. base+15 take the even and then the odd halves of blocks base/2 .. +7
    // (a last partial run of 16 keeps the identity order)
    const int i = b - p.S * nbig, base = i & ~15;
    const int b2 = base + 16 <= p.S * nsmall ? base + 2 * (i & 7) + ((i >> 3) & 1) : i;
    const int r = b2 / nsmall, j = b2 - r * nsmall;
    const int c0 = 64 * nbig + 32 * j;
    diag_run<T, kDiagN, 2, false>(p, DiagWork{r, 0, c0, min(32, p.H - c0), nbig == 0 && j == 0},
                                  sm.small);
  }
}

template <typename T, int NS, int SPL, bool kScalarA>
static void launch_diag(const PrefillParams& p, hipStream_t s) {
  constexpr int CH = DiagCfg<NS, SPL>::CH;
  const dim3 grid(p.G * diag_blocks_per_group(p.H, p.G, CH), p.S);
  hipLaunchKernelGGL((k_diag_scan<T, NS, SPL, kScalarA>), grid, dim3(256), 0, s, p);
}

// CUs of the current device (cached per device; 256 on MI355X).
static int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The Mamba1 scan's grid: the uniform one (64-channel workgroups), or the mixed one when
// it spreads the work more evenly over the CUs.  Model: workgroups land one per CU per pass
// in grid order, a CU's time is its large workgroups plus kSmallCost per small one.
constexpr double kSmallCost = 0.6;
struct Mamba1Grid {
  bool mixed;
  int nbig, nsmall;
};
static Mamba1Grid mamba1_grid(int S, int H, int cus) {
  const int nu = S * ((H + 63) / 64);
  const double t_uni = double((nu + cus - 1) / cus);
  const int nbig = 2 * (H / 160), nsmall = (H - 64 * nbig + 31) / 32;
  if (S <= 0 || nsmall <= 0) return {false, 0, 0};
  const int big = S * nbig, total = S * (nbig + nsmall);
  double t_mix = 0.0;
  for (int c = 0; c < cus && c < total; ++c) {
    const int nb_c = c < big ? (big - 1 - c) / cus + 1 : 0;
    const int ns_c = c < total ? (total - 1 - c) / cus + 1 - nb_c : 0;
    t_mix = std::max(t_mix, nb_c + kSmallCost * ns_c);
  }
  return {t_mix < t_uni - 0.05, nbig, nsmall};
}

bool diag_mixed_grid(bool scalar_a, int S, int H, int G, int N) {
  return !scalar_a && N == kDiagN && G == 1 && mamba1_grid(S, H, device_cus()).mixed;
}

template <typename T>
static hipError_t launch_diag_t(const PrefillParams& p, bool scalar_a, hipStream_t s) {
  if (diag_mixed_grid(scalar_a, p.S, p.H, p.G, p.N)) {
    const Mamba1Grid mg = mamba1_grid(p.S, p.H, device_cus());
    hipLaunchKernelGGL((k_diag_scan_mixed<T>), dim3(p.S * (mg.nbig + mg.nsmall)), dim3(256), 0, s,
                       p, mg.nbig, mg.nsmall);
    return hipSuccess;
  }
  if (!scalar_a && p.N == kDiagN) launch_diag<T, 16, SSD_DIAG_SPL, false>(p, s);
  else if (scalar_a && p.N == 16) launch_diag<T, 16, 4, true>(p, s);
  else if (scalar_a && p.N == 128) launch_diag<T, 128, 8, true>(p, s);
  else return hipErrorInvalidValue;   // the plan admits no other dstate
  return hipSuccess;
}

hipError_t launch_diag_prefill(int in_dtype, bool scalar_a, const PrefillParams& p, hipStream_t s,
                               void* const* events) {
  record_event(events, 0, s);
  const hipError_t e = in_dtype == SSD_BF16 ? launch_diag_t<bf16_t>(p, scalar_a, s)
                                            : launch_diag_t<float>(p, scalar_a, s);
  if (e != hipSuccess) return e;
  record_event(events, 1, s);
  return hipGetLastError();
}

}  // namespace ssd
